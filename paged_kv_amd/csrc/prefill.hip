// Varlen flash-attention prefill on quantized Q/K/V for gfx950.
//
// Computes O = softmax(sm_scale * Dequant(Q) Dequant(K)^T + causal mask) Dequant(V)
// (Ascend "KvQuantSparseFlashAttention" formula; FlashInfer's ragged batch
// prefill; aiter's fp8 flash_attn_func with q/k/v descales; PaddleNLP's Sage
// attention over a varlen batch with per-block int8 Q/K).
//
// Work split: one workgroup (4 waves) per (sequence, q head, 128-query tile)
// on a 1-D grid whose order (pf_work_item) starts the tiles with the most
// visible keys first and keeps the q heads of one kv head on one XCD.  Each
// wave owns 32 queries and streams 64-key tiles staged in LDS by direct
// loads (a ring of two stages, or of three K stages when fp8 V is widened
// through registers).
//
// Per key tile and wave:
//   S^T = K Q^T          fp8 codes widened to fp16 (exact) and f16 16x16x32
//                        MFMAs (an fp32-exact sum; the fp8 16x16x128 MFMA sums
//                        its 128 products to only ~2^-12 of sum |q_d k_d|,
//                        available as a separate Q/K form), or two int8
//                        16x16x64 (exact, accumulated onto the bits of a float
//                        bias so no conversion is needed); the codes' scales
//                        and sm_scale*log2(e) are folded into one multiplier
//                        per tile;
//   online softmax       one fma + exp2 per score against a lagging reference
//                        max, moved (tile max across the 4 lanes that hold one
//                        query; O and l rescale) only when a tile's partial
//                        row sum leaves [0, 2^14]; row sums by dot2 over the
//                        fp16 P fed to the PV MFMA;
//   O^T += V^T P^T       fp16 16x16x32 MFMA; P is rounded to fp16, fp8 V codes
//                        are widened to fp16 (exactly) when staged into LDS.
//                        With fp16 V^T the operands are read from LDS one
//                        16-dim block at a time inside the product: holding
//                        them all across the softmax costs 64 VGPRs, and with
//                        them the third workgroup per CU.  The fp8-V forms
//                        run two workgroups per CU either way and read them
//                        while the softmax runs (8% faster there).
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
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Workgroup shape: each wave owns 32 queries; 4 waves (128 queries).  With
// fp16 V^T the kernel fits three workgroups per CU (at most 168 VGPRs, 48 KB
// of LDS in a two-stage ring); the fp8-V forms hold more registers and a
// third K stage and run two.  More resident waves matter more here than a
// deeper ring: one workgroup per CU runs the varlen workload 1.7x slower than
// two, and three are 6% faster than two with three stages.  (8 waves / 256
// queries halve the K/V tile traffic but leave one workgroup per CU, whose
// barriers nothing covers: measured slower on the varlen workload, about even
// on the long one.  8 waves of 16 queries each, two workgroups per CU, read
// the K and V tiles from LDS twice as often per query: 7-10% slower.)
template <int D>
struct PfShape {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BM = WAVES * 32;  // queries per workgroup
};
constexpr int PF_BN = 64;   // keys per tile
constexpr int PF_NST = 3;   // K stages of the fp8-V ring (two tiles in flight)
constexpr int PF_XCD_CUS = 32;  // CUs per XCD
constexpr float PF_LN2 = 0.69314718055994530942f;
// buffer descriptor word 3 for untyped 32-bit accesses
constexpr int PF_RSRC_W3 = 0x00020000;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS tile geometry.  Rows are unpadded; the 16-byte chunk c of row r sits at
// chunk position c ^ swizzle(r), while the direct loads (64 lanes x 16
// contiguous bytes) write linearly.  On this LDS (measured) a 16-byte read
// is served in four passes of 16 lanes -- each half-wave split by the parity
// of lane bits 2..4 -- across 64 four-byte banks, and a 16-byte write in
// eight passes of 8 consecutive lanes across 32 banks.  The swizzles give the
// 16 lanes of every K and V^T read pass 16 distinct 16-byte bank groups, and
// the two rows of every 8-lane pass of the fp8 V^T stores opposite halves.
template <int D, bool V_F8>
struct PfGeo {
  static constexpr int K_CH = D / 16;                  // chunks per K row (codes)
  static constexpr int KBYTES = PF_BN * D;             // one K tile
  static constexpr int VBYTES = D * PF_BN * 2;         // one V^T tile (fp16, 128-byte rows)
  static constexpr int WAVES = PfShape<D>::WAVES;
  static constexpr int THREADS = PfShape<D>::THREADS;
  static constexpr int NKD = KBYTES / 1024 / WAVES;                // K direct loads per wave per tile
  static constexpr int NVD = V_F8 ? 0 : VBYTES / 1024 / WAVES;     // V^T direct loads per wave per tile
  static_assert(NKD >= 1 && (V_F8 || NVD >= 1), "every wave takes a share of each tile");
  static constexpr int NST = V_F8 ? PF_NST : 2;     // K (and DMA'd V^T) stages of the ring
  static constexpr int DIST = NST - 1;              // tiles in flight ahead of the current one
  static constexpr int NV_ST = V_F8 ? 2 : NST;      // V^T stages (fp8 V is widened through registers)
  static constexpr int VC = V_F8 ? D * PF_BN / 16 / THREADS : 0;     // fp8 V^T u32x4 per thread
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = NST * KBYTES;
  static constexpr int LDS = V_OFF + NV_ST * VBYTES;
  static ATTNQ_DEV int ksw(int r) { return D == 128 ? (((r >> 1) & 1) | (((r >> 2) & 1) << 2)) : (((r >> 2) & 1) << 1); }
  static ATTNQ_DEV int vsw(int r) { return r & 7; }
  // token-major fp16 V rows (paged form): D / 8 chunks per row.  Even
  // swizzles: a transposed-read pass (8 rows x 2 chunks of each) covers all
  // 16 (D = 128) or, per row parity, all 8 (D = 64) chunk positions.
  static ATTNQ_DEV int tsw(int r) { return D == 128 ? (r & 7) << 1 : ((r >> 1) & 3) << 1; }
};

ATTNQ_DEV __amdgpu_buffer_rsrc_t pf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, PF_RSRC_W3);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (they complete in issue order), N a compile-time constant.
template <int N>
ATTNQ_DEV void pf_wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4]=7, lgkmcnt[11:8]=15
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Workgroup barrier of the LDS ring.  This wave's LDS stores have completed
// (lgkmcnt 0) and its direct loads were waited for explicitly above it.  A
// __syncthreads() would add a release fence, which waits for every vector
// memory operation, including the next tile's direct loads still in flight.
ATTNQ_DEV void pf_barrier() {
  // gfx9 s_waitcnt: lgkmcnt[11:8]=0, vmcnt[3:0]+[15:14] and expcnt[6:4] at maximum
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  // no LDS access of this wave moves above the barrier (no wait is needed)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 16 fp8 codes (one u32x4) -> 16 fp16 values (exact), two u32x4.
ATTNQ_DEV void pf_widen_fp8(const u32x4 w, u32x4& lo, u32x4& hi) {
  lo[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, false));
  lo[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, true));
  lo[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, false));
  lo[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, true));
  hi[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2], 1.0f, false));
  hi[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[2], 1.0f, true));
  hi[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[3], 1.0f, false));
  hi[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[3], 1.0f, true));
}

// 8 fp8 codes (two dwords) -> 8 fp16 values (exact).
ATTNQ_DEV v8h pf_widen8(uint32_t w0, uint32_t w1) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Direct loads of one tile: K rows into the K stage and (fp16 V) V^T rows into
// the V stage; this wave's share is blocks [wave*N, wave*N + N) of 1 KB.
template <int D, bool V_F8>
ATTNQ_DEV void pf_dma(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, const uint32_t* kvo,
                      const uint32_t* vvo, uint32_t k_soff, uint32_t v_soff, uint8_t* kdst, uint8_t* vdst) {
  using G = PfGeo<D, V_F8>;
#pragma unroll
  for (int j = 0; j < G::NKD; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(kdst + j * 1024), 16, kvo[j], k_soff, 0, 0);
#pragma unroll
  for (int j = 0; j < G::NVD; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(vdst + j * 1024), 16, vvo[j], v_soff, 0, 0);
}

// Transposed LDS read (ds_read_b64_tr_b16): in each 16-lane group, lane
// 4k + q names 4 consecutive 16-bit values of row k; lane n receives value n
// of the 4 rows (column n of the 4 x 16 block).
typedef __fp16 pf_h4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
ATTNQ_DEV u32x2 pf_read_tr16(const uint8_t* p) {
  const pf_h4 v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) pf_h4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// A tile whose fp16 partial row sum (16 scores per lane) stays at or below
// this keeps the lagging reference max: every p is then <= 2^14, well inside
// fp16, and O / l need no rescale.
constexpr float PF_TILE_SUM_MAX = 16384.0f;

// int8 scores are accumulated onto the bits of this float (1.5 * 2^23)
constexpr float PF_BIAS = 12582912.0f;
constexpr int PF_BIAS_BITS = 0x4B400000;

// Work item (sequence b, q head h, query tile counted from the sequence end
// ty) of linear workgroup id lin; ntiles query tiles per (sequence, head).
// Workgroups are dealt round-robin to the 8 XCDs (id mod 8), each with its own
// L2.  When the kv heads split evenly over the XCDs, XCD x takes the kv heads
// hk = x (mod 8) and runs its share in blocks of tblk query tiles, the tiles
// with the most keys first (so that no long workgroup starts late).  Inside a
// block it goes stream by stream ((sequence, kv head)), then tile by tile,
// the q heads of one kv head side by side: workgroups that run together read
// the same K/V tiles, which the XCD's L2 then serves once.  Otherwise tiles
// with the most keys go first over all (sequence, head) pairs.  Both maps are
// bijections of [0, batch*hq*ntiles).
ATTNQ_DEV void pf_work_item(const PrefillArgs& a, int ntiles, int lin, int& b, int& h, int& ty) {
  if ((a.hkv & 7) == 0) {
    const int grp = a.hq / a.hkv;
    const int xcd = lin & 7, j = lin >> 3;
    const int nstream = a.batch * (a.hkv >> 3);  // (sequence, kv head) streams of this XCD
    const int tb = max(1, min(a.tblk, ntiles));
    const int blk = j / (nstream * tb * grp);
    const int t0 = blk * tb;
    const int tl = min(tb, ntiles - t0);          // the last block may be short
    const int r = j - blk * (nstream * tb * grp);
    const int st = r / (tl * grp), r2 = r - st * (tl * grp);
    const int t = r2 / grp;
    b = st % a.batch;
    h = (xcd + 8 * (st / a.batch)) * grp + (r2 - t * grp);
    ty = t0 + t;
  } else {
    const int nbh = a.batch * a.hq;
    const int bh = lin % nbh;
    b = bh / a.hq;
    h = bh - b * a.hq;
    ty = lin / nbh;
  }
}

template <int D, int QM, bool V_F8, bool O_BF16, bool PAGED>
__global__ __launch_bounds__(PfShape<D>::THREADS, V_F8 ? 2 : 3) void k_prefill(const PrefillArgs a) {
  using G = PfGeo<D, V_F8>;
  constexpr bool QK_F8 = QM == PF_Q_FP8 || QM == PF_Q_FP8_MFMA8;  // fp8 codes
  constexpr bool QK_I8 = !QK_F8;                             // int8 QK MFMA
  constexpr bool Q_RAW = QM == PF_Q_RAW_F16 || QM == PF_Q_RAW_BF16;  // Q quantized here
  static_assert(!PAGED || (QK_F8 && V_F8), "the paged form reads fp8 K and V pages");
  constexpr bool V_EARLY = V_F8;  // V^T operands read before the softmax
  static_assert(!PAGED || G::DIST == 2, "the paged form keeps the V pages of tile kt+1 from the K loads of kt+2");
  // the DMA ring, then 4 floats for the block-amax exchange of a raw Q
  __shared__ __attribute__((aligned(16))) uint8_t smem[G::LDS + 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  int b, h, ty;
  pf_work_item(a, (int)gridDim.x / (a.batch * a.hq), (int)blockIdx.x, b, h, ty);
  b = __builtin_amdgcn_readfirstlane(b);
  h = __builtin_amdgcn_readfirstlane(h);
  const int tile = (int)gridDim.x / (a.batch * a.hq) - 1 - ty;
  const int q0 = clampi(a.cu_q[b], 0, a.total_q), q1 = clampi(a.cu_q[b + 1], q0, a.total_q);
  // keys: a ragged range of K / V^T, or (PAGED) the sequence's page list, its
  // length (pages - 1) * page_size + the last page's fill (FlashInfer's paged
  // layout: kv_indptr, kv_indices, kv_last_page_len)
  int k0 = 0, Lk;
  int p0 = 0, npg = 0;
  if constexpr (PAGED) {
    p0 = __builtin_amdgcn_readfirstlane(a.kv_indptr[b]);
    npg = __builtin_amdgcn_readfirstlane(max(0, a.kv_indptr[b + 1] - p0));
    Lk = npg > 0 ? (npg - 1) * a.page_size + clampi(a.kv_last[b], 0, a.page_size) : 0;
  } else {
    k0 = clampi(a.cu_k[b], 0, a.total_k);
    Lk = clampi(a.cu_k[b + 1], k0, a.total_k) - k0;
  }
  // lengths beyond the host-given maxima would address past the padded V^T
  // rows and the scale arrays: clamp (a broken precondition, not a fault)
  const int Lq = min(q1 - q0, a.max_q);
  Lk = __builtin_amdgcn_readfirstlane(min(Lk, a.max_k));
  constexpr int BM = PfShape<D>::BM;
  const int qs = tile * BM;
  if (qs >= Lq) return;
  const int hk = __builtin_amdgcn_readfirstlane(h / (a.hq / a.hkv));
  const int off = Lk - Lq;  // bottom-right causal alignment
  int kend = Lk;
  if (a.causal) kend = min(Lk, qs + BM + off);
  const int n_kt = kend > 0 ? (kend + PF_BN - 1) / PF_BN : 0;
  const int wq0 = qs + wave * 32;  // first query of this wave
  // keys visible to this wave's last query end here (wave-uniform)
  const int wave_kend = a.causal ? min(Lk, wq0 + 32 + off) : Lk;

  // ---- Q operand (B of S^T = K Q^T): lane (n, g) holds d in [g*D/4, (g+1)*D/4)
  constexpr int QB = D / 4;  // codes (bytes) per lane and row
  v4i qop[2][2];             // [query block][16-byte half]
  int lim[2];                // per-lane key limit (exclusive) of query row qb
  u32x4 qx[2][Q_RAW ? QB / 8 : 1];  // raw 16-bit Q: QB values per row, 8 per chunk
  // raw Q rows of this workgroup's 128 queries (this head): the range ends
  // at the sequence's last query
  const int qstride = a.hq * D * 2;  // bytes per token
  const __amdgpu_buffer_rsrc_t qrs =
      pf_rsrc(static_cast<const uint8_t*>(a.q) + ((long)(q0 + qs) * a.hq + h) * D * (Q_RAW ? 2 : 1),
              Q_RAW ? (uint32_t)((min(Lq - qs, BM) - 1) * qstride + D * 2) : 0u);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = wq0 + qb * 16 + n;
    qop[qb][0] = qop[qb][1] = v4i{0, 0, 0, 0};
    if constexpr (Q_RAW) {
      // unconditional buffer loads; rows past the sequence end read as zeros
      // (they stay out of the block amax and encode to 0)
#pragma unroll
      for (int c = 0; c < QB / 8; ++c)
        qx[qb][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  qrs, (uint32_t)((row - qs) * qstride + (g * QB + c * 8) * 2), 0u, 0));
    } else if (row < Lq) {
      const uint8_t* src = static_cast<const uint8_t*>(a.q) + ((long)(q0 + row) * a.hq + h) * D + g * QB;
      qop[qb][0] = *reinterpret_cast<const v4i*>(src);
      if constexpr (QB == 32) qop[qb][1] = *reinterpret_cast<const v4i*>(src + 16);
    }
    lim[qb] = a.causal ? min(Lk, row + off + 1) : Lk;
  }
  // Q has landed before the first tile load is issued.  Otherwise the
  // compiler, unable to tell the Q loads from the tile loads in flight in the
  // loop, drains the next tile's loads before every tile's first MFMA.  (A raw
  // Q is waited for after the first tiles' loads are issued, below.)
  if constexpr (!Q_RAW) pf_wait_vm<0>();
  // fp8 codes summed exactly: the lane's QB codes of each query row as
  // QB/8 fp16 operands of 8 (codes 8m .. 8m+7 of its bytes)
  v8h q16[2][QB / 8];
  if constexpr (QM == PF_Q_FP8) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int m = 0; m < QB / 8; ++m)
        q16[qb][m] = pf_widen8((uint32_t)qop[qb][m >> 1][2 * (m & 1)], (uint32_t)qop[qb][m >> 1][2 * (m & 1) + 1]);
  }

  float q_sc = 1.0f;
  if constexpr (Q_RAW) {
  } else if constexpr (QK_I8) {
    q_sc = a.q_scale[((long)b * a.hq + h) * a.nblk_q + (wq0 >> 7)];  // 128-query block
  } else {
    q_sc = a.q_scale[h];
  }
  const float k_sc_head = QK_I8 ? 0.0f : a.k_scale[hk];
  // int8: one scale per 128-key block, read through the scalar cache (the
  // constant address space) so no vector-memory wait joins the tile loads
  const __attribute__((address_space(4))) float* k_sc_blk =
      (const __attribute__((address_space(4))) float*)(uintptr_t)(a.k_scale + ((long)b * a.hkv + hk) * a.nblk_k);
  float base_fold = a.sm_scale_log2 * q_sc;

  // ---- tile sources as buffer descriptors: K rows of this (sequence, kv head)
  // with the range ending at the last key (rows past it arrive as zeros), and
  // the padded V^T block of this (sequence, kv head).
  const long kstride = (long)a.hkv * D;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + ((long)k0 * a.hkv + hk) * D;
  // PAGED: the whole cache from this kv head's first row on (host-checked
  // below 2 GiB); each row's page offset goes into its lane's load offset
  const __amdgpu_buffer_rsrc_t krs =
      PAGED ? pf_rsrc(kbase, (uint32_t)((long)a.num_pages * a.page_size * kstride - (long)hk * D))
            : pf_rsrc(kbase, Lk > 0 ? (uint32_t)((Lk - 1) * kstride + D) : 0u);
  const long vrow = (long)a.s_pad * (V_F8 ? 1 : 2);  // bytes per V^T row
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + ((long)b * a.hkv + hk) * D * vrow;
  const __amdgpu_buffer_rsrc_t vrs = pf_rsrc(vbase, (uint32_t)(D * vrow));

  // per-lane byte offsets of the direct loads: wave w fills 1 KB blocks
  // w*N + j of the K (and V^T) stage; lane i of a block writes its chunk i
  uint32_t kvo[G::NKD];
  int krow[G::NKD];  // PAGED: the tile row of each load (kvo then holds its chunk offset)
#pragma unroll
  for (int j = 0; j < G::NKD; ++j) {
    const int blk = wave * G::NKD + j;
    const int r = blk * (1024 / D) + lane / G::K_CH;
    const int c = (lane % G::K_CH) ^ G::ksw(r);
    krow[j] = r;
    kvo[j] = PAGED ? (uint32_t)(c * 16) : (uint32_t)(r * kstride + c * 16);
  }
  uint32_t vvo[G::NVD > 0 ? G::NVD : 1];
#pragma unroll
  for (int j = 0; j < G::NVD; ++j) {
    const int blk = wave * G::NVD + j;
    const int r = blk * 8 + lane / 8;
    const int c = (lane % 8) ^ G::vsw(r);
    vvo[j] = (uint32_t)(r * vrow + c * 16);
  }
  // PAGED: cache rows by page.  The (at most 4: page sizes are multiples of
  // 16) pages that hold keys [64t, 64t + 64) are read through the scalar
  // cache, with indices clamped into the sequence's page list and page ids
  // into [0, num_pages).  A row then sits at byte (page * page_size + slot) *
  // kstride of the cache (plus the kv head's offset).
  const __attribute__((address_space(4))) int32_t* kv_ix =
      (const __attribute__((address_space(4))) int32_t*)(uintptr_t)(a.kv_indices + p0);
  const int ps = a.page_size;
  // With page_size a multiple of 64 every tile lies inside one page: its
  // rows are one wave-uniform page offset plus the row's own offset.
  const bool one_page = ps % PF_BN == 0;
  struct TilePages {
    int id[4];
    int x0;         // position of key 64t inside the first page
    uint32_t base;  // one_page: byte offset of key 64t in the cache
  };
  auto tile_pages = [&](int t) {
    TilePages tp;
    const int first = (t * PF_BN) / ps;
    tp.x0 = t * PF_BN - first * ps;
    if (one_page) {
      tp.id[0] = clampi(kv_ix[min(first, npg - 1)], 0, a.num_pages - 1);
      tp.id[1] = tp.id[2] = tp.id[3] = tp.id[0];
      tp.base = (uint32_t)(tp.id[0] * ps + tp.x0) * (uint32_t)kstride;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) tp.id[i] = clampi(kv_ix[min(first + i, npg - 1)], 0, a.num_pages - 1);
      tp.base = 0;
    }
    return tp;
  };
  // byte offset of tile row r (r < 64) in the cache
  auto row_off = [&](const TilePages& tp, int r) -> uint32_t {
    if (one_page) return tp.base + (uint32_t)r * (uint32_t)kstride;
    const int x = tp.x0 + r;
    const int pi = (x >= ps) + (x >= 2 * ps) + (x >= 3 * ps);
    const int page = pi == 0 ? tp.id[0] : pi == 1 ? tp.id[1] : pi == 2 ? tp.id[2] : tp.id[3];
    return (uint32_t)(page * ps + (x - pi * ps)) * (uint32_t)kstride;
  };
  // fp8 V: 16 codes per load, widened to fp16 on the way into LDS.  Ragged:
  // V^T rows (16 keys of one d).  PAGED: token rows (16 d of one key); rows
  // past the last key are zeros (a stale slot of the last page may hold NaN
  // codes, and NaN times p = 0 is still NaN).
  u32x4 vreg[G::VC > 0 ? G::VC : 1];
  auto vload = [&](int t, const TilePages& tp) {
    static_for<0, G::VC>([&](auto ci) {
      constexpr int c = decltype(ci)::value;
      const int idx = threadIdx.x + c * G::THREADS;
      if constexpr (PAGED) {
        const int r = idx / (D / 16), cc = idx % (D / 16);
        vreg[c] = u32x4{0, 0, 0, 0};
        if (t * PF_BN + r < Lk)
          vreg[c] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.v) + (long)hk * D +
                                                    row_off(tp, r) + cc * 16);
      } else {
        vreg[c] = *reinterpret_cast<const u32x4*>(vbase + (long)t * PF_BN + (idx >> 2) * vrow + (idx & 3) * 16);
      }
    });
  };
  auto vstore = [&](int stage) {
    static_for<0, G::VC>([&](auto ci) {
      constexpr int c = decltype(ci)::value;
      const int idx = threadIdx.x + c * G::THREADS;
      u32x4 lo, hi;
      pf_widen_fp8(vreg[c], lo, hi);
      if constexpr (PAGED) {
        // token-major fp16 rows of D * 2 bytes, 16-byte chunk j of row r at
        // chunk position j ^ tsw(r).  Half of each 8-lane write pass stores
        // its odd chunk first, so every pass covers 8 distinct positions.
        const int r = idx / (D / 16), cc = idx % (D / 16);
        uint8_t* row = smem + G::V_OFF + stage * G::VBYTES + r * (2 * D);
        const int sw = D == 128 ? (cc >> 2) & 1 : r & 1;
        *reinterpret_cast<u32x4*>(row + ((2 * cc + sw) ^ G::tsw(r)) * 16) = sw ? hi : lo;
        *reinterpret_cast<u32x4*>(row + ((2 * cc + 1 - sw) ^ G::tsw(r)) * 16) = sw ? lo : hi;
      } else {
        const int r = idx >> 2, j = idx & 3;
        uint8_t* row = smem + G::V_OFF + stage * G::VBYTES + r * 128;
        *reinterpret_cast<u32x4*>(row + ((2 * j) ^ G::vsw(r)) * 16) = lo;
        *reinterpret_cast<u32x4*>(row + ((2 * j + 1) ^ G::vsw(r)) * 16) = hi;
      }
    });
  };
  // PAGED: the direct-load offsets of tile t, returning the soffset.  One
  // page per tile: the page offset goes in the soffset, and rows past the
  // last key read the page's stale slots (their scores are masked by
  // select, which NaN codes cannot pass).  Else each row's page offset is
  // in its lane's offset, and rows past the last key address beyond the
  // range (zeros).
  auto kvo_paged = [&](int t, const TilePages& tp, uint32_t (&vo)[G::NKD]) -> uint32_t {
    if (one_page) {
#pragma unroll
      for (int j = 0; j < G::NKD; ++j) vo[j] = (uint32_t)krow[j] * (uint32_t)kstride + kvo[j];
      return tp.base;
    }
#pragma unroll
    for (int j = 0; j < G::NKD; ++j) vo[j] = t * PF_BN + krow[j] < Lk ? row_off(tp, krow[j]) + kvo[j] : 0x80000000u;
    return 0u;
  };

  const uint32_t ktile_bytes = (uint32_t)(PF_BN * kstride);
  // this wave's 1 KB blocks of stage st
  auto kdst = [&](int st) { return smem + G::K_OFF + st * G::KBYTES + wave * G::NKD * 1024; };
  auto vdst = [&](int st) { return smem + G::V_OFF + st * G::VBYTES + wave * G::NVD * 1024; };

  // per-lane LDS read offsets (swizzled); kb / db add whole 16-row blocks
  const int kr0 = (D == 128 ? n * 128 + (((2 * g) ^ G::ksw(n)) * 16) : n * 64 + ((g ^ G::ksw(n)) * 16));
  const int kr1 = n * 128 + (((2 * g + 1) ^ G::ksw(n)) * 16);  // D == 128 only
  const int vr0 = n * 128 + ((g ^ G::vsw(n)) * 16);
  const int vr1 = n * 128 + (((4 + g) ^ G::vsw(n)) * 16);
  // PAGED: transposed reads of token-major V (ds_read_b64_tr_b16).  In each
  // 16-lane group g, lane 4k + q names row 4g + k (+ 16h + 32ks) and the 4
  // values of d = 16db + 4q..; lane n receives d = 16db + n of those 4 rows:
  // keys 32ks + 16h + 4g + 0..3, the keys of P slots 4h..4h+3 of the lane.
  // Chunk 2db + q/2 of the row sits at (2db + q/2) ^ t, t = tsw(row), i.e.
  // at 2(db ^ t/2) + (q/2 ^ t%2): the block part is db ^ t/2 in bits 5 and up
  // of the offset, below the row's, so block db's offset is vtr0 ^ 32db.
  const int vtr_row = 4 * g + (n >> 2), vtr_q = n & 3;
  const int vtr_t = G::tsw(vtr_row);
  const int vtr0 = vtr_row * (2 * D) + (vtr_t >> 1) * 32 + (((vtr_q >> 1) ^ (vtr_t & 1)) * 16) + (vtr_q & 1) * 8;

  // ---- accumulators
  v4f oacc[D / 16][2];
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = v4f{0.f, 0.f, 0.f, 0.f};
  // reference max (log2 units) per query row; -inf until set, so the first
  // tile's p are inf/NaN and force the exact path
  float m_ref[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};              // lane-local partial row sums
  const v2h ones = v2h{(_Float16)1.0f, (_Float16)1.0f};

  // ---- prologue: the first DIST tiles in flight
  constexpr int NPEND = G::NKD + G::NVD;  // direct loads per wave per tile
  TilePages tp_v{};  // PAGED: the pages of the next V tile to load
  if constexpr (Q_RAW && !V_F8) {
    // unconditional, so that one wait below counts them: loads past the last
    // key read zeros (range-checked descriptors) into stages no tile uses
    pf_dma<D, V_F8>(krs, vrs, kvo, vvo, 0u, 0u, kdst(0), vdst(0));
    if constexpr (G::DIST == 2) pf_dma<D, V_F8>(krs, vrs, kvo, vvo, ktile_bytes, PF_BN * 2, kdst(1), vdst(1));
  } else if (PAGED && n_kt > 0) {
    const TilePages tp0 = tile_pages(0);
    uint32_t vo[G::NKD];
    uint32_t so = kvo_paged(0, tp0, vo);
    pf_dma<D, V_F8>(krs, vrs, vo, vvo, so, 0u, kdst(0), vdst(0));
    vload(0, tp0);
    if (n_kt > 1) {
      tp_v = tile_pages(1);
      so = kvo_paged(1, tp_v, vo);
      pf_dma<D, V_F8>(krs, vrs, vo, vvo, so, 0u, kdst(1), vdst(1));
    }
  } else if (n_kt > 0) {
    pf_dma<D, V_F8>(krs, vrs, kvo, vvo, 0u, 0u, kdst(0), vdst(0));
    if constexpr (V_F8) vload(0, TilePages{});
    if (G::DIST == 2 && n_kt > 1) pf_dma<D, V_F8>(krs, vrs, kvo, vvo, ktile_bytes, PF_BN * 2, kdst(1), vdst(1));
  }
  if constexpr (Q_RAW) {
    // This workgroup's 128 queries are one quantization block (128 tokens
    // from the sequence start): scale = amax/127 over the block, codes =
    // clamp(rint(x / scale), -127, 127), the codes and scale attn_quant_qk
    // writes in INT8_PER_BLOCK mode (same arithmetic, same helpers).  The Q
    // loads went out before the first tiles' loads: wait for them only.
    if constexpr (V_F8) pf_wait_vm<0>();
    else pf_wait_vm<G::DIST * NPEND>();
    constexpr bool BF = QM == PF_Q_RAW_BF16;
    float m = 0.0f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int c = 0; c < QB / 8; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          m = fmaxf(m, fabsf(h16_to_f32(qx[qb][c][e] & 0xffffu, BF)));
          m = fmaxf(m, fabsf(h16_to_f32(qx[qb][c][e] >> 16, BF)));
        }
    m = wave_max(m);
    float* s_amax = reinterpret_cast<float*>(smem + G::LDS);
    if (lane == 0) s_amax[wave] = m;
    pf_barrier();
    const float amax = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));
    const float scale = amax == 0.0f ? 1.0f : amax / 127.0f;
    if (a.q_scale_out != nullptr && threadIdx.x == 0)
      a.q_scale_out[((long)b * a.hq + h) * a.nblk_q + tile] = scale;
    const float rs = 1.0f / scale;
    auto encode = [&](auto fast_c) {
      constexpr bool FAST = decltype(fast_c)::value;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int c = 0; c < QB / 8; ++c)
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t bits = (qx[qb][c][2 * w + j / 2] >> (16 * (j & 1))) & 0xffffu;
              const float xv = h16_to_f32(bits, BF);
              const uint32_t code = (uint32_t)int8_encode(FAST ? quot_by_recip_i8(xv, scale, rs) : xv / scale) & 0xffu;
              word |= code << (8 * j);
            }
            qop[qb][c >> 1][(c & 1) * 2 + w] = (int)word;
          }
    };
    if (scale >= QUOT_MIN_SCALE) encode(std::true_type{});  // uniform
    else encode(std::false_type{});
    q_sc = scale;
    base_fold = a.sm_scale_log2 * q_sc;
  }

  int kst = 0;  // K (and DMA'd V^T) stage of tile kt
  int m_grid = -126;  // int8: every finite m_ref is a multiple of 2^m_grid (wave-uniform)
  for (int kt = 0; kt < n_kt; ++kt) {
    if constexpr (V_F8) vstore(kt & 1);
    // PAGED: the pages of tile kt+DIST, read through the scalar cache before
    // the barrier's wait covers them
    TilePages tp_k{};
    if constexpr (PAGED) {
      if (kt + G::DIST < n_kt) tp_k = tile_pages(kt + G::DIST);
    }
    // tile kt landed (with three stages, tile kt+1's direct loads may still be
    // in flight)
    if (G::DIST == 2 && kt + 1 < n_kt) pf_wait_vm<NPEND>();
    else pf_wait_vm<0>();
    pf_barrier();
    // the stage of tile kt+DIST was last read in tile kt-1: every wave is past it
    if constexpr (V_F8) {
      if (kt + 1 < n_kt) vload(kt + 1, tp_v);
    }
    if (kt + G::DIST < n_kt) {
      const int st2 = G::NST == 2 ? 1 - kst : (kst == 0 ? 2 : kst - 1);
      if constexpr (PAGED) {
        uint32_t vo[G::NKD];
        const uint32_t so = kvo_paged(kt + G::DIST, tp_k, vo);
        pf_dma<D, V_F8>(krs, vrs, vo, vvo, so, 0u, kdst(st2), vdst(st2));
        tp_v = tp_k;
      } else {
        pf_dma<D, V_F8>(krs, vrs, kvo, vvo, (uint32_t)(kt + G::DIST) * ktile_bytes, (uint32_t)(kt + G::DIST) * (PF_BN * 2),
                        kdst(st2), vdst(st2));
      }
    }
    const int cur = kst;
    kst = kst == G::NST - 1 ? 0 : kst + 1;
    const int kfirst = kt * PF_BN;
    if (kfirst >= wave_kend) continue;  // every key of this tile is masked for this wave
    const uint8_t* sk = smem + G::K_OFF + cur * G::KBYTES;
    const uint8_t* sv = smem + G::V_OFF + (V_F8 ? (kt & 1) : cur) * G::VBYTES;

    // ---- S^T = K Q^T (raw code products).  The MFMA blocks run at raised
    // wave priority: when both waves of a SIMD are ready, the one entering its
    // matrix section issues first and the other's softmax fills the gaps.
    __builtin_amdgcn_s_setprio(1);
    float s[4][2][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const v4i ka = *reinterpret_cast<const v4i*>(sk + kb * 16 * D + kr0);
      v4i kb2 = v4i{0, 0, 0, 0};
      if constexpr (QB == 32) kb2 = *reinterpret_cast<const v4i*>(sk + kb * 16 * D + kr1);
      v8h kw16[QB / 8];  // this key's codes as fp16, the layout of q16
      if constexpr (QM == PF_Q_FP8) {
#pragma unroll
        for (int m = 0; m < QB / 8; ++m) {
          const v4i src = m < 2 ? ka : kb2;
          kw16[m] = pf_widen8((uint32_t)src[2 * (m & 1)], (uint32_t)src[2 * (m & 1) + 1]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if constexpr (QK_I8) {
          // The integer sum s (|s| < 2^21) is accumulated onto the bits of
          // PF_BIAS = 1.5 * 2^23: the result's bits are those of the float
          // PF_BIAS + s, exactly (ulp 1 on [2^23, 2^24)), with no conversion.
          // The bias leaves the exp2 argument exactly (see the fold below).
          // Each element passes an empty asm first: reading elements of an
          // int MFMA result one by one otherwise makes this compiler read
          // element 0 for all four.
          v4i acc = v4i{PF_BIAS_BITS, PF_BIAS_BITS, PF_BIAS_BITS, PF_BIAS_BITS};
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka, qop[qb][0], acc, 0, 0, 0);
          if constexpr (QB == 32) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(kb2, qop[qb][1], acc, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            int bits = acc[r];
            asm("" : "+v"(bits));
            s[kb][qb][r] = __builtin_bit_cast(float, bits);
          }
        } else {
          const v8i kop = v8i{ka[0], ka[1], ka[2], ka[3], kb2[0], kb2[1], kb2[2], kb2[3]};
          const v8i qo = v8i{qop[qb][0][0], qop[qb][0][1], qop[qb][0][2], qop[qb][0][3],
                             qop[qb][1][0], qop[qb][1][1], qop[qb][1][2], qop[qb][1][3]};
          v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
          if constexpr (QM == PF_Q_FP8_MFMA8) {
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, qo, acc, 0, 0, 0, 0, 0, 0);
          } else {
            // the lane's QB codes of key n and query n, 8 at a time: the same
            // dims for both operands of each f16 MFMA (the order of the terms
            // over the MFMAs does not change the sum)
#pragma unroll
            for (int m = 0; m < QB / 8; ++m)
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kw16[m], q16[qb][m], acc, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) s[kb][qb][r] = acc[r];
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // V^T operands of a 16-dim block
    auto vread = [&](int db, v8h* dst) {
      if constexpr (PAGED) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int vtr = vtr0 ^ (32 * db);
          const u32x2 lo = pf_read_tr16(sv + vtr + (32 * ks) * (2 * D));
          const u32x2 hi = pf_read_tr16(sv + vtr + (32 * ks + 16) * (2 * D));
          dst[ks] = __builtin_bit_cast(v8h, u32x4{lo[0], lo[1], hi[0], hi[1]});
        }
      } else {
        dst[0] = *reinterpret_cast<const v8h*>(sv + db * 2048 + vr0);
        dst[1] = *reinterpret_cast<const v8h*>(sv + db * 2048 + vr1);
      }
    };
    v8h vop[V_EARLY ? D / 16 : 1][2];
    if constexpr (V_EARLY) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) vread(db, vop[db]);
    }

    float fold;
    if constexpr (QK_I8)
      fold = base_fold * k_sc_blk[kt >> 1];
    else
      fold = base_fold * k_sc_head;
    // int8: the scores are PF_BIAS + s.  The fold is rounded to 22
    // significant bits (a relative change of at most 2^-23, twice fp32's own
    // rounding of the scale product), so that bfold = PF_BIAS * fold is exact
    // and a multiple of 2^grid_t.  While every reference m_ref is a multiple
    // of 2^m_grid with m_grid >= grid_t, bfold + m_ref is exact too, and
    // fma(PF_BIAS + s, fold, -(bfold + m_ref)) is s * fold - m_ref rounded
    // once: the exp2 argument of an unbiased score.
    float bfold = 0.0f;
    int grid_t = -125;
    bool big = false;   // a grid above 1 would shift p too far: no bias
    if constexpr (QK_I8) {
      const uint32_t fb = (__builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, fold)) + 2u) & ~3u;
      fold = __builtin_bit_cast(float, fb);
      bfold = PF_BIAS * fold;
      grid_t = max((int)((fb >> 23) & 0xffu) - 126, -125);
      big = grid_t > 0;
    }

    // ---- mask (tiles that cross the causal diagonal or the sequence end):
    // the fold is applied first and the scaled logit of a key past the row's
    // limit becomes -inf by select, so the mask holds for any fold
    // (sm_scale <= 0, scales of either sign) and NaN garbage in a masked key
    // cannot leak.  Such a tile then continues with a unit fold and no bias.
    // An int8 tile whose fold is too large for the bias grid takes the bias
    // off instead (same loop, nothing masked) and keeps its fold.
    const bool need_mask = kfirst + PF_BN > min(Lk, wq0 + off + 1);
    if (need_mask || big) {
      // masked: s * fold or -inf, then a unit fold.  Large fold, no key
      // masked: PF_BIAS + s - PF_BIAS = s exactly (the two lie within a
      // factor 2 of each other), and the tile keeps its fold, so its exp2
      // argument is still s * fold - m_ref rounded once.
      const float fm = need_mask ? fold : 1.0f;
      const float bm = need_mask ? bfold : PF_BIAS;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kfirst + kb * 16 + 4 * g + r;
            s[kb][qb][r] = key < lim[qb] ? __builtin_fmaf(s[kb][qb][r], fm, -bm) : -INFINITY;
          }
      if (need_mask) fold = 1.0f;
      bfold = 0.0f;
    }
    // a biased tile whose fold needs a coarser reference grid than the rows'
    // references are on goes through the exact path, which moves them up to it
    bool bump = false;
    if (QK_I8 && !need_mask && !big && grid_t > m_grid) {
      m_grid = grid_t;
      bump = true;
    }

    // ---- online softmax against a lagging reference max.  Common path:
    // p = exp2(s * fold - m_ref), no max.  A lane whose fp16 partial row sum
    // of this tile exceeds 2^14 (or overflowed), or a row without a reference
    // yet, sends the whole wave through the exact path: tile max, move the
    // reference, rescale O and l, recompute p.
    v8h pk[2][2];
    float lt[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float neg_m = -(bfold + m_ref[qb]);
      lt[qb] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * ks + e / 4][qb][e % 4], fold, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * ks + e / 4][qb][e % 4 + 1], fold, neg_m));
          const v2h ph = __builtin_convertvector(v2f{p0, p1}, v2h);
          pk[qb][ks][e] = ph[0];
          pk[qb][ks][e + 1] = ph[1];
          lt[qb] = __builtin_amdgcn_fdot2(ph, ones, lt[qb], false);
        }
    }
    // NaN-safe: !(x <= bound) also catches inf/NaN partial sums
    const bool redo = !(lt[0] <= PF_TILE_SUM_MAX) || !(lt[1] <= PF_TILE_SUM_MAX);
    if (__ballot(redo) || bump) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        // the row's largest scaled logit in this tile (masked keys are -inf)
        float m = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) m = fmaxf(m, __builtin_fmaf(s[kb][qb][r], fold, -bfold));
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        float m_new = fmaxf(m_ref[qb], m);
        if constexpr (QK_I8) {
          // up to the next multiple of 2^m_grid (a float at or above 2^23 of
          // them already is one; -inf stays)
          const float t = __builtin_ldexpf(m_new, -m_grid);
          if (fabsf(t) < 0x1p23f) m_new = __builtin_ldexpf(__builtin_ceilf(t), m_grid);
        }
        const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_ref[qb] - m_new);
        m_ref[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) oacc[db][qb] *= alpha;
        const float neg_m = m_new == -INFINITY ? -bfold : -(bfold + m_new);
        lt[qb] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * ks + e / 4][qb][e % 4], fold, neg_m));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * ks + e / 4][qb][e % 4 + 1], fold, neg_m));
            const v2h ph = __builtin_convertvector(v2f{p0, p1}, v2h);
            pk[qb][ks][e] = ph[0];
            pk[qb][ks][e + 1] = ph[1];
            lt[qb] = __builtin_amdgcn_fdot2(ph, ones, lt[qb], false);
          }
      }
    }
    l_run[0] += lt[0];
    l_run[1] += lt[1];

    // ---- O^T += V^T P^T
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      v8h vl[2];
      if constexpr (!V_EARLY) vread(db, vl);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(V_EARLY ? vop[db][ks] : vl[ks], pk[qb][ks], oacc[db][qb], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  }
  // No direct load may outlive the workgroup's LDS.  The last tile waits for
  // every load it issued; this covers a workgroup whose loop never ran (no
  // visible key: n_kt == 0) after the raw-Q prologue issued its tiles anyway.
  pf_wait_vm<0>();

  // ---- epilogue: O = O^T / l, lse = (m + log2 l) * ln 2
  // V descale: fp8 codes, or fp16 values that carry one (the widened codes)
  const float vsc = a.v_scale && !a.v_chan ? a.v_scale[hk] : 1.0f;
  // per-channel descales: output column d is scaled by v_scale[b][hk][d]
  const float* vch = a.v_chan ? a.v_scale + ((long)b * a.hkv + hk) * D : nullptr;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = l_run[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int row = wq0 + qb * 16 + n;
    if (row >= Lq) continue;
    const bool any = l != 0.0f;  // a visible key (a NaN sum stays NaN)
    const float inv = any ? vsc / l : 0.0f;
    const long obase = ((long)(q0 + row) * a.hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int d0 = db * 16 + 4 * g;
      v4f o4 = oacc[db][qb] * inv;
      if (vch) o4 *= *reinterpret_cast<const v4f*>(vch + d0);
      u32x2 w;
      if constexpr (O_BF16) {  // hardware round-to-nearest-even
        w[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{o4[0], o4[1]}, v2bf));
        w[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{o4[2], o4[3]}, v2bf));
      } else {
        w[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{o4[0], o4[1]}, v2h));
        w[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{o4[2], o4[3]}, v2h));
      }
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.o) + obase + d0) = w;
    }
    if (a.lse && g == 0)
      a.lse[(long)h * a.total_q + q0 + row] = any ? (m_ref[qb] + __log2f(l)) * PF_LN2 : -INFINITY;
  }
}

template <int D, int QM, bool F8, bool PAGED = false>
static bool launch_t(const PrefillArgs& args, bool o_bf16, int max_seqlen_q, hipStream_t s) {
  const int tiles = (max_seqlen_q + PfShape<D>::BM - 1) / PfShape<D>::BM;
  if ((long)args.batch * args.hq * tiles > 0x7FFFFFFFL) return false;
  PrefillArgs a = args;
  // blocks of (workgroups resident on an XCD) / group tiles: about that many
  // workgroups of one (sequence, kv head) stream run side by side on an XCD
  // (three per CU with fp16 V^T, two with fp8 V at head_dim 128)
  static const int per_cu = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_prefill<D, QM, F8, true, PAGED>, PfShape<D>::THREADS,
                                                     0) != hipSuccess || n < 1)
      n = 2;
    return n;
  }();
  a.tblk = max(1, PF_XCD_CUS * per_cu / (a.hq / a.hkv));
  dim3 grid((unsigned)(a.batch * a.hq * tiles));
  if (o_bf16)
    hipLaunchKernelGGL((k_prefill<D, QM, F8, true, PAGED>), grid, dim3(PfShape<D>::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((k_prefill<D, QM, F8, false, PAGED>), grid, dim3(PfShape<D>::THREADS), 0, s, a);
  return hipGetLastError() == hipSuccess;
}

template <int D, int QM>
static bool launch_v(const PrefillArgs& a, bool v_fp8, bool o_bf16, int max_seqlen_q, hipStream_t s) {
  return v_fp8 ? launch_t<D, QM, true>(a, o_bf16, max_seqlen_q, s) : launch_t<D, QM, false>(a, o_bf16, max_seqlen_q, s);
}

template <int D>
static bool launch_q(const PrefillArgs& a, int q_mode, bool v_fp8, bool o_bf16, int max_seqlen_q, hipStream_t s) {
  switch (q_mode) {
    case PF_Q_FP8: return launch_v<D, PF_Q_FP8>(a, v_fp8, o_bf16, max_seqlen_q, s);
    case PF_Q_FP8_MFMA8: return launch_v<D, PF_Q_FP8_MFMA8>(a, v_fp8, o_bf16, max_seqlen_q, s);
    case PF_Q_I8: return launch_v<D, PF_Q_I8>(a, v_fp8, o_bf16, max_seqlen_q, s);
    case PF_Q_RAW_F16: return launch_v<D, PF_Q_RAW_F16>(a, v_fp8, o_bf16, max_seqlen_q, s);
    case PF_Q_RAW_BF16: return launch_v<D, PF_Q_RAW_BF16>(a, v_fp8, o_bf16, max_seqlen_q, s);
    default: return false;
  }
}

bool launch_prefill(const PrefillArgs& a, int head_dim, int q_mode, bool v_fp8, bool o_bf16,
                    int max_seqlen_q, hipStream_t s) {
  if (max_seqlen_q <= 0 || a.batch <= 0) return true;
  return head_dim == 128 ? launch_q<128>(a, q_mode, v_fp8, o_bf16, max_seqlen_q, s)
                         : launch_q<64>(a, q_mode, v_fp8, o_bf16, max_seqlen_q, s);
}

template <int D>
static bool launch_paged_d(const PrefillArgs& a, int q_mode, bool o_bf16, int max_seqlen_q, hipStream_t s) {
  return q_mode == PF_Q_FP8_MFMA8 ? launch_t<D, PF_Q_FP8_MFMA8, true, true>(a, o_bf16, max_seqlen_q, s)
                                  : launch_t<D, PF_Q_FP8, true, true>(a, o_bf16, max_seqlen_q, s);
}

bool launch_prefill_paged(const PrefillArgs& a, int head_dim, int q_mode, bool o_bf16, int max_seqlen_q,
                          hipStream_t s) {
  if (max_seqlen_q <= 0 || a.batch <= 0) return true;
  if (q_mode != PF_Q_FP8 && q_mode != PF_Q_FP8_MFMA8) return false;
  return head_dim == 128 ? launch_paged_d<128>(a, q_mode, o_bf16, max_seqlen_q, s)
                         : launch_paged_d<64>(a, q_mode, o_bf16, max_seqlen_q, s);
}

}  // namespace attnq
