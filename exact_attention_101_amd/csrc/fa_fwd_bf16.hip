// bf16 FlashAttention forward for gfx950 (MI355X).
//
// The method (FlashAttention v1 post, DeepSchool #630, sections «Тайлинг
// (Tiling)» and «Онлайн-Softmax»): each workgroup owns a block of BR query
// rows and streams the key/value blocks of its head past them through LDS.
// For every K/V block it forms the scores on the matrix cores, updates a
// running row maximum m and a running denominator l, rescales the partial
// output by exp(m_old - m_new) when the maximum grows, and accumulates P V.
// Only O and the per-row log-sum-exp leave the chip (section «Итог»; the
// FlashAttention-3 summary, section «Resumo do FlashAttention»).  The two
// matrix products with the softmax between them, and the layout change in
// between, are the shape named in paragraph 2 of "Оптимизируйте
// производительность с FlashAttention-4".
//
// gfx950 mapping:
//   * workgroup = BR = 256 query rows: 4 waves, one per SIMD, each owning
//     64 query rows as two 32-row MFMA blocks, so every K or V fragment a
//     wave reads from LDS feeds two MFMAs: LDS reads per FLOP are half of
//     what 32-row waves need, and LDS traffic is what the matrix cores
//     otherwise wait on and what the power budget goes to.  The variable-
//     length configuration uses 8 waves of 32 rows, two per SIMD (more
//     issue slots for the window masks), the masked one 4 waves of 32 rows
//     (128 rows; two workgroups per CU);
//   * K and V blocks of BT = 64 keys go from HBM/L2 straight into LDS with
//     buffer_load_dwordx4 ... lds (no register staging), into two K and two
//     V stage arrays (distinct arrays, so the compiler can tell the
//     in-flight copies from the stages being read).  Compute steps take
//     BC = 32 keys, so copies and the workgroup barrier come every second
//     step;
//   * scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16: the accumulator column is the query, so each
//     lane holds the 16 scores of one query per 32-key step, and a row's
//     two halves sit in lanes l and l ^ 32;
//   * Q lives in registers as the B operand for the whole kernel; the
//     contraction over d is permuted so that lane half h holds the
//     contiguous d-range [h*D/2, (h+1)*D/2);
//   * K rows are loaded in sigma order (fa_common.h), so the fp32 score
//     accumulator, converted to bf16, is directly the B operand of
//     O^T = V^T P^T; V stays in its [key][d] layout in LDS and the A operand
//     (V^T) is read with the transposing ds_read_b64_tr_b16;
//   * softmax in fp32 registers in the log2 domain: p = exp2(S*c - m) with
//     c = |scale| * log2(e) (one FMA + v_exp_f32 per score), fp32 row sums;
//   * a three-stage software pipeline overlaps the two matrix products with
//     the softmax inside each wave (the intra-group overlap of the
//     FlashAttention-3 summary, section «Assincronia: sobreposição de GEMM e
//     Softmax»): step b issues, slot by slot, one MFMA of the scores of
//     block b+1, one MFMA of O += P(b-1) V(b-1) and one pair of
//     p = exp2(S c - m) of block b, so the vector unit works while the
//     matrix core runs.  The order is pinned with scheduling barriers;
//   * the running maximum m is a reference value, not necessarily the exact
//     maximum: any m gives the same softmax (the shift cancels between
//     numerator and denominator), so P is first formed with the m already
//     held.  Only if a lane's sum of the block's p exceeds 2^TAU (some score
//     rose more than TAU = 8 log2 units above m; also inf / NaN) does the
//     wave take the exact step: row maximum of the block, move m, rescale O
//     and l, form P again.  All p stay in [0, 2^TAU]; block 0 sets m from
//     its exact row maximum, so the common path computes no maximum at all;
//   * LDS layouts are chosen so every MFMA operand read is free of bank
//     conflicts: K rows are padded by one 16-byte slot, V rows XOR their
//     64-byte segments with the key's position in its group of 4;
//   * VL (variable-length batches and sliding windows, FlashAttention-3
//     summary, section «Comentários no Hacker News»): the causal
//     configuration with per-sequence row offsets, a key range [lo, hi]
//     per workgroup (tiles before lo are never loaded; K / V are addressed
//     from lo's tile), window masks in the masked blocks, and the XCDs fed
//     by KV head rather than by sequence.  A row that has seen no key keeps
//     m = -inf and forms P against 0; the first block in which it sees a
//     key takes the exact step;
//   * MK (arbitrary visibility masks, same section): before its loop each
//     workgroup ORs (and ANDs) its rows' mask words into a list of the
//     64-key tiles some row sees, each flagged if every row sees all of it;
//     the copies follow the list, so work scales with the visible tiles.
//     Each lane's mask words of a listed tile are fetched with the tile's K
//     copy unless the tile is whole for the workgroup, and a block is
//     masked score by score only where some row of the wave misses a key.
#include "fa_common.h"

#ifndef FA_PAIR1
#define FA_PAIR1 1
#endif

#ifndef FA_PERSIST
#define FA_PERSIST 1
#endif


namespace fa {

namespace {

constexpr int BT = 64;                  // keys per K / V stage (copy tile)
constexpr int BC = 32;                  // keys per compute step
constexpr float TAU_EXP2 = 256.0f;      // 2^TAU, TAU = 8 (log2 units)

// Waves of a workgroup: NQB 32-row query blocks per wave and NW waves,
// BR = 32 NQB NW query rows (NQB = 2, NW = 4: 256 rows, one wave per SIMD;
// NQB = 1, NW = 8: 256 rows, two waves per SIMD; NQB = 2, NW = 2: 128 rows,
// two workgroups per CU).
template <int NQB, int NW = 8 / NQB>
struct Waves {
  static constexpr int NWAVE = NW;
  static constexpr int QPW = 32 * NQB;            // query rows per wave
  static constexpr int NTHR = 64 * NWAVE;
  static constexpr int BR = NWAVE * QPW;          // query rows per workgroup
};

typedef __attribute__((ext_vector_type(4))) short i16x4_t;

template <bool V>
struct Tag {
  static constexpr bool value = V;
};
template <int V>
struct Int {
  static constexpr int value = V;
};

template <int D, int NWAVE>
struct Geo {
  static constexpr int NCH = D / 8;                // 16-byte chunks per row
  static constexpr int NDB = D / 32;               // 32-wide d blocks
  static constexpr int NKS = D / 16;               // QK^T MFMA k-steps
  // K: rows padded to NCH + 1 slots (16 bytes each): 16 consecutive rows at
  // the same chunk land in 16 different 4-bank groups.
  static constexpr int KSL = NCH + 1;
  static constexpr int KSLOTS = BT * KSL;
  static constexpr int KINS = KSLOTS / 64;         // 64-lane copies per tile
  static constexpr int KPW = (KINS + NWAVE - 1) / NWAVE;   // per wave, max
  // V: unpadded rows, 64-byte segments XOR-swizzled.
  static constexpr int VSLOTS = BT * NCH;
  static constexpr int VINS = VSLOTS / 64;
  static constexpr int VPW = VINS / NWAVE;
  static_assert(KSLOTS % 64 == 0 && VSLOTS % (64 * NWAVE) == 0,
                "copy tiling");
};

// Segment swizzle of V row r: the 4 rows read together by one transposing
// read (r = 4a + R) must use 4 different 16-bank groups.
template <int D>
__device__ __forceinline__ int vx(int r) {
  if constexpr (D == 128) {
    return r & 3;
  } else {
    return (r >> 1) & 1;
  }
}

// Transposing LDS read.  In each group of 16 lanes, lane 4R + j supplies the
// address of 4 consecutive 16-bit elements; output lane i of the group gets
// element i % 4 of the chunks of lanes 4R + i / 4, for R = 0..3.
__device__ __forceinline__ i16x4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Lane l and lane l ^ 32 hold the two halves of the same query's row.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// O^T += V^T P^T with the accumulator held in accumulation registers (the
// 128 fp32 values of O per lane for D = 128 do not fit in the vector
// registers next to Q, S and P).  The library is built with VGPR-form
// MFMAs for the compiler's own MFMA instructions (the scores, which the
// vector unit reads); this one is written out so that its accumulator stays
// in AGPRs without being moved around.  The compiler does not see that the
// statement is an MFMA, so every other access of O is fenced by hand: reads
// after acc_read_fence(), writes followed by acc_write_fence().  The ISA
// test in the test suite checks the compiled kernels for accesses of an
// accumulator within the MFMA's latency.
__device__ __forceinline__ void mfma_pv_acc(const bf16x8_t& a,
                                            const bf16x8_t& b,
                                            f32x16_t& acc) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+a"(acc)
               : "v"(a), "v"(b));
}
// Wait states between the last mfma_pv_acc and any other access of its
// accumulator: an 8-pass MFMA result needs 11 before a VALU or memory
// instruction may read or overwrite it; 3 x s_nop 7 give 24.
__device__ __forceinline__ void acc_read_fence() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}
// Wait states between a VALU write of an accumulator and the next
// mfma_pv_acc reading it as its C operand.
__device__ __forceinline__ void acc_write_fence() {
  asm volatile("s_nop 4" ::: "memory");
}

// One 64-lane copy of 16 bytes per lane from `rsrc` (+ voffset + soffset
// bytes; soffset is wave-uniform) into LDS at `dst` + 16 * lane.  Offsets
// past the descriptor's size read zeros.
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc,
                                            const uint4* dst,
                                            uint32_t voffset,
                                            uint32_t soffset = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)(dst), 16, voffset,
      soffset, 0, 0);
}

template <int D, bool CAUSAL, int NQB, bool VL = false, bool MK = false,
          int NW = 8 / NQB>
__global__ void __launch_bounds__((Waves<NQB, NW>::NTHR), 1)
fwd_bf16_kernel(const FwdArgs a_arg) {
  constexpr int NWAVE = Waves<NQB, NW>::NWAVE;
  constexpr int QPW = Waves<NQB, NW>::QPW;
  constexpr int BR = Waves<NQB, NW>::BR;
  // Rows may see no key of a block, or none at all (windows, masks).
  constexpr bool VM = VL || MK;
  using G = Geo<D, NWAVE>;
  __shared__ uint4 Ks0[G::KSLOTS];
  __shared__ uint4 Ks1[G::KSLOTS];
  __shared__ uint4 Vs0[G::VSLOTS];
  __shared__ uint4 Vs1[G::VSLOTS];
  // MK: the key tiles some row of the workgroup sees, in order (tl: tile
  // index, bit 15 set if every row sees all of the tile's keys below NK),
  // their count (tl_n), and while they are gathered a bit per tile that
  // some row sees (tfl) and one per tile that some row does not see whole
  // (tfp).
  constexpr int NTL = MK ? MASK_MAX_NK / BT : 1;
  __shared__ uint16_t tl[NTL];
  __shared__ uint32_t tfl[MK ? NTL / 32 : 1];
  __shared__ uint32_t tfp[MK ? NTL / 32 : 1];
  __shared__ int tl_n[1];

  const int tid0 = threadIdx.x;
  const int wave0 = __builtin_amdgcn_readfirstlane(tid0 >> 6);   // uniform

  // Work units: (batch, head, query block), one per workgroup, except in
  // the persistent launch of the dense non-causal forward (a.persist: N a
  // multiple of BR, one workgroup per CU), where a workgroup takes units
  // blockIdx.x, blockIdx.x + gridDim.x, ... (all of equal work).  There the
  // last copy steps of a unit copy the next unit's first K and V tiles into
  // the stages its prologue would fill, and the next unit's Q loads are
  // issued before this unit's epilogue, so the next unit starts without
  // waiting for memory (and without a workgroup launch).
  constexpr bool PS = !CAUSAL && !VL && !MK;
  const int nunits = PS && a_arg.persist ? a_arg.B * a_arg.H * a_arg.nqb
                                         : static_cast<int>(gridDim.x);
  uint4 qraw[NQB][G::NKS];              // Q of the unit, as loaded
  bool have = false;                    // its Q loads and first tiles issued
  // (One trip, known at compile time, unless PS.)
  for (int unit = blockIdx.x, trip = 0; PS ? unit < nunits : trip < 1;
       unit += static_cast<int>(gridDim.x), ++trip) {
  // The arguments are read again for every unit (scalar-cache hits), so
  // that none of them is held in a register across the main loop.
  typedef const __attribute__((address_space(4))) FwdArgs KArgs;
  KArgs* ap = (KArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  if constexpr (PS) asm volatile("" : "+s"(ap));
  KArgs& a = *ap;
  // PS: the lane index is also taken again for every unit, so that the
  // per-lane offsets derived from it are formed per unit instead of being
  // held (and spilled) across the unit loop.
  int tid = tid0;
  if constexpr (PS)
    tid = 64 * wave0 +
          __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int lane = tid & 63;
  const int wave = wave0;
  const int li = lane & 31;             // MFMA column / row-in-block
  const int h = lane >> 5;              // lane half
  int bh, qblk;
  if constexpr (VL) {
    // Sequences differ in length, so no XCD may own whole sequences:
    // workgroups go to the 8 XCDs in turn, and XCD x takes the KV heads
    // hk = x (mod 8) of every sequence (its query heads together, sharing
    // K and V in that XCD's L2), longest-running query blocks first.  With
    // Hkv not a multiple of 8, consecutive workgroups take consecutive
    // (sequence, head) pairs.
    const int L = unit;
    if (a.xcd_chunk) {
      const int x = L & 7;
      int t = L >> 3;
      const int g = t % a.group;
      t /= a.group;
      const int hpx = a.Hkv >> 3;
      const int hk_l = t % hpx;
      t /= hpx;
      const int bb = t % a.B;
      qblk = a.nqb - 1 - t / a.B;
      bh = bb * a.H + (hk_l * 8 + x) * a.group + g;
    } else {
      bh = L % (a.B * a.H);
      qblk = a.nqb - 1 - L / (a.B * a.H);
    }
  } else {
    map_work(unit, nunits, a.B * a.H, a.nqb, CAUSAL, a.xcd_chunk, bh, qblk);
  }
  const int b = bh / a.H;
  const int hq = bh % a.H;
  const int hk = hq / a.group;
  const int q0 = qblk * BR;
  const int qw0 = q0 + wave * QPW;      // first query row of this wave
  // This lane's query rows: qw0 + 32 j + li for query block j < NQB.

  // NQ query rows and NK keys in this (batch, head), or in this sequence of
  // a variable-length batch: rows of Q / O start at row qrow0 of the
  // tensor, rows of K / V at krow0.  VL: query i sees key j iff
  // (wl < 0 or j >= i + off - wl) and (wr < 0 or j <= i + off + wr), with
  // off = NK - NQ (bottom-right alignment).
  int NQ, NK, off = 0, wl = -1, wr = -1;
  int64_t qrow0, krow0;
  if constexpr (VL) {
    const int q_beg = a.cu_q[b];
    const int k_beg = a.cu_k[b];
    NQ = a.cu_q[b + 1] - q_beg;
    NK = a.cu_k[b + 1] - k_beg;
    // A sequence whose offsets leave the packed tensors is skipped; so are
    // query blocks past its last row (the whole workgroup, before any
    // barrier).
    if (q_beg < 0 || NQ < 0 || q_beg + NQ > a.total_q || k_beg < 0 ||
        NK < 0 || k_beg + NK > a.total_k || q0 >= NQ)
      return;
    off = NK - NQ;
    wl = a.left;
    wr = a.right;
    qrow0 = static_cast<int64_t>(hq) * a.total_q + q_beg;
    krow0 = static_cast<int64_t>(hk) * a.total_k + k_beg;
  } else if constexpr (MK) {
    NQ = a.total_q;
    NK = a.total_k;
    qrow0 = (static_cast<int64_t>(b) * a.H + hq) * NQ;
    krow0 = (static_cast<int64_t>(b) * a.Hkv + hk) * NK;
  } else {
    NQ = NK = a.N;
    qrow0 = (static_cast<int64_t>(b) * a.H + hq) * a.N;
    krow0 = (static_cast<int64_t>(b) * a.Hkv + hk) * a.N;
  }
  // Keys [kv_begin, kv_begin + kv_end) are streamed (kv_begin is a multiple
  // of BT); blocks and tiles below count from kv_begin.
  int kv_begin = 0, kv_end;
  if constexpr (VL) {
    const int i1 = min(NQ, q0 + BR) - 1;
    const int lo = wl < 0 ? 0 : max(0, q0 + off - wl);
    const int hi = wr < 0 ? NK - 1 : min(NK - 1, i1 + off + wr);
    kv_begin = hi < lo ? 0 : (lo / BT) * BT;
    kv_end = hi < lo ? 0 : hi + 1 - kv_begin;
  } else {
    kv_end = CAUSAL ? min(NK, q0 + BR) : NK;   // last key needed + 1
  }

  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow0 * D;
  const uint16_t* kp =
      static_cast<const uint16_t*>(a.k) + (krow0 + kv_begin) * D;
  const uint16_t* vp =
      static_cast<const uint16_t*>(a.v) + (krow0 + kv_begin) * D;

  // ---- Q -> registers (B operand of S^T = K Q^T), NQB query blocks ----
  // All of the wave's Q loads are issued here; the fragments move to the
  // accumulation registers only after the prologue's tile copies are
  // issued (below), so the Q loads and the copies wait together once,
  // instead of each load waiting in turn.
  bf16x8_t qf[NQB][G::NKS];
  // Q rows qwx + 32 j + li (j < NQB) of the nq rows at qpx.
  auto load_q = [&](const uint16_t* qpx, int qwx, int nq) {
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      const int row = qwx + 32 * j + li;
      const bool ok = row < nq;
      const uint16_t* src = qpx + static_cast<int64_t>(ok ? row : nq - 1) * D +
                            h * (D / 2);
#pragma unroll
      for (int s = 0; s < G::NKS; ++s)
        qraw[j][s] = keep_if(ldg16(src + 8 * s), ok);
    }
  };
  if (!have) load_q(qp, qw0, NQ);

  // PS: the next unit's Q rows, K and V (false when there is none).  The
  // unit index is taken opaquely, so that this is formed where it is used
  // (the last copy steps, the loop's end) and not held across the loop.
  auto next_unit = [&](const uint16_t*& nq, const uint16_t*& nk,
                       const uint16_t*& nv) {
    int nu = unit + static_cast<int>(gridDim.x);
    asm volatile("" : "+s"(nu));
    if (nu >= nunits) return false;
    int bh2, qb2;
    map_work(nu, nunits, a.B * a.H, a.nqb, CAUSAL, a.xcd_chunk, bh2, qb2);
    const int b2 = bh2 / a.H;
    const int hk2 = (bh2 % a.H) / a.group;
    nq = static_cast<const uint16_t*>(a.q) +
         (static_cast<int64_t>(bh2) * a.N + qb2 * BR) * D;
    const int64_t k2 = (static_cast<int64_t>(b2) * a.Hkv + hk2) * a.N * D;
    nk = static_cast<const uint16_t*>(a.k) + k2;
    nv = static_cast<const uint16_t*>(a.v) + k2;
    return true;
  };
  auto settle_q = [&]() {
    const uint32_t flip = a.neg ? 0x80008000u : 0u;
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
#pragma unroll
      for (int s = 0; s < G::NKS; ++s) {
        uint4 u = qraw[j][s];
        u.x ^= flip; u.y ^= flip; u.z ^= flip; u.w ^= flip;
        qf[j][s] = as_bf16x8(u);
        // Q is only ever an MFMA operand, which MFMA reads from
        // accumulation registers directly: keep it there and leave the
        // vector registers to the scores and probabilities.
        asm volatile("" : "+a"(qf[j][s]));
      }
    }
  };

  // ---- MK: the 64-key tiles some row of the workgroup sees ----
  // Each wave ORs the mask rows q0 + wave, q0 + wave + NWAVE, ... word by
  // word (lane L holds words 4 L .. 4 L + 3 of each 256-word chunk, four
  // rows in flight), marks the tiles with a visible key in tfl, and wave 0
  // turns the marks into the ordered list tl.  Bits past NK are ignored.
  int ntl = 0;
  const uint32_t* mrow[NQB];              // this lane's mask rows
  if constexpr (MK) {
    const uint32_t* mp = a.mask + b * a.mask_bs + hq * a.mask_hs;
    const int W = a.mw;
    const int nt = (NK + BT - 1) / BT;
    const int ntw = (nt + 31) / 32;
    const int r1 = min(NQ, q0 + BR);
    for (int i = tid; i < ntw; i += Waves<NQB, NW>::NTHR) {
      tfl[i] = 0u;
      tfp[i] = 0u;
    }
#pragma unroll
    for (int j = 0; j < NQB; ++j)
      mrow[j] = mp + static_cast<int64_t>(min(qw0 + 32 * j + li, NQ - 1)) * W;
    __syncthreads();
    const uint32_t tail = (NK & 31) ? (1u << (NK & 31)) - 1u : ~0u;
    // Rows of 16-byte aligned words (W % 4 == 0 and an aligned mask) are
    // read 16 bytes per lane, sixteen rows in flight; others word by word.
    const bool vec = (W & 3) == 0 &&
                     (reinterpret_cast<uintptr_t>(mp) & 15) == 0;
    for (int c0 = 0; c0 < W; c0 += 256) {
      const int j0 = c0 + 4 * lane;
      uint32_t acc[4] = {0u, 0u, 0u, 0u};       // OR over the rows
      uint32_t all[4] = {~0u, ~0u, ~0u, ~0u};   // AND over the rows
      if (vec) {
        for (int r = q0 + wave; r < r1; r += 16 * NWAVE) {
          uint4 x[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int rr = r + u * NWAVE;
            const uint32_t* rp =
                mp + static_cast<int64_t>(rr < r1 ? rr : r) * W;
            x[u] = (j0 < W) ? *reinterpret_cast<const uint4*>(rp + j0)
                            : make_uint4(0u, 0u, 0u, 0u);
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            acc[0] |= x[u].x;
            acc[1] |= x[u].y;
            acc[2] |= x[u].z;
            acc[3] |= x[u].w;
            all[0] &= x[u].x;
            all[1] &= x[u].y;
            all[2] &= x[u].z;
            all[3] &= x[u].w;
          }
        }
      } else {
        for (int r = q0 + wave; r < r1; r += 4 * NWAVE) {
          uint32_t x[4][4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int rr = r + u * NWAVE;
            const uint32_t* rp =
                mp + static_cast<int64_t>(rr < r1 ? rr : r) * W;
#pragma unroll
            for (int k = 0; k < 4; ++k)
              x[u][k] = (j0 + k < W) ? rp[j0 + k] : 0u;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              acc[k] |= x[u][k];
              all[k] &= x[u][k];
            }
        }
      }
      // Bits past NK are ignored: never seen, never missing.
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (j0 + k == W - 1) {
          acc[k] &= tail;
          all[k] |= ~tail;
        }
      }
      // Words 4 L .. 4 L + 3 are tiles 2 L' and 2 L' + 1 (L' = j0 / 4).
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int t = j0 / 2 + e;
        if (t < nt) {
          if ((acc[2 * e] | acc[2 * e + 1]) != 0u)
            atomicOr(&tfl[t >> 5], 1u << (t & 31));
          if ((all[2 * e] & all[2 * e + 1]) != ~0u)
            atomicOr(&tfp[t >> 5], 1u << (t & 31));
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      // Lane L gathers words 2 L and 2 L + 1 of tfl (up to 4096 tiles).
      const uint32_t f0 = (2 * lane < ntw) ? tfl[2 * lane] : 0u;
      const uint32_t f1 = (2 * lane + 1 < ntw) ? tfl[2 * lane + 1] : 0u;
      const uint32_t p0 = (2 * lane < ntw) ? tfp[2 * lane] : ~0u;
      const uint32_t p1 = (2 * lane + 1 < ntw) ? tfp[2 * lane + 1] : ~0u;
      const int cnt = __builtin_popcount(f0) + __builtin_popcount(f1);
      int incl = cnt;
#pragma unroll
      for (int dlt = 1; dlt < 64; dlt <<= 1) {
        const int y = __shfl_up(incl, dlt);
        if (lane >= dlt) incl += y;
      }
      int pos = incl - cnt;
      for (uint32_t f = f0; f; f &= f - 1u) {
        const int b = __builtin_ctz(f);
        tl[pos++] = static_cast<uint16_t>(64 * lane + b +
                                          (((p0 >> b) & 1u) ? 0 : 0x8000));
      }
      for (uint32_t f = f1; f; f &= f - 1u) {
        const int b = __builtin_ctz(f);
        tl[pos++] = static_cast<uint16_t>(64 * lane + 32 + b +
                                          (((p1 >> b) & 1u) ? 0 : 0x8000));
      }
      if (lane == 63) tl_n[0] = incl;
    }
    __syncthreads();
    ntl = __builtin_amdgcn_readfirstlane(tl_n[0]);
  }
  // MK: the list is read through two 64-entry windows in registers (lane L
  // holds entries 64 w0 + L and 64 (w0 + 1) + L), so that a tile's entry
  // comes from v_readlane and not from an LDS read the wave must wait for.
  // Positions are asked for in increasing order; the windows move on (once
  // every 64 tiles) just before the barrier that precedes each copy step,
  // which also waits for that LDS read, so a lookup has no read behind it
  // (one could only be waited for together with every fragment read in
  // flight).
  int win0 = 0, win1 = 0, w0 = 0;
  if constexpr (MK) {
    win0 = tl[lane];
    win1 = tl[64 + lane];
  }
  // MK: move the windows on until they hold position tmax.
  auto advance_list = [&](int tmax) {
    while ((tmax >> 6) >= w0 + 2) {           // rare: next window
      win0 = win1;
      const int i = 64 * (w0 + 2) + lane;
      win1 = i < NTL ? tl[i] : 0;
      ++w0;
    }
  };
  // Entry of tile position t < ntl (MK), 64 w0 <= t < 64 (w0 + 2).
  auto entry = [&](int t) -> int {
    return __builtin_amdgcn_readlane((t >> 6) == w0 ? win0 : win1, t & 63);
  };
  // First key of tile position t (MK: of the t-th listed tile; positions
  // past the list are virtual, their copies read nothing), and (MK) whether
  // every row of the workgroup sees all of its keys below NK.
  auto tkv = [&](int t) {
    if constexpr (MK)
      return t < ntl ? (entry(t) & 0x7FFF) * BT : NK;
    else
      return t * BT;
  };
  auto tfull = [&](int t) {
    if constexpr (MK)
      return t >= ntl || (entry(t) & 0x8000) != 0;
    else
      return true;
  };

  // ---- per-lane byte offsets of this wave's tile copies ----
  // K copy j (j = wave + 4 i) fills slots 64 j .. 64 j + 63: lane L writes
  // slot 64 j + L = row * KSL + chunk; pad slots re-read the last chunk.
  // Offsets are below 2^15: copies 2 i2 and 2 i2 + 1 share a register, and
  // a copy past the first four (the last window, one wave) computes its
  // offsets when issued.
  auto k_offset = [&](int i) {
    const int slot = 64 * (wave + NWAVE * i) + lane;
    const int row = slot / G::KSL;
    const int ch = min(slot - row * G::KSL, G::NCH - 1);
    return static_cast<uint32_t>((row * D + ch * 8) * 2);
  };
  // Copies with a precomputed offset (four, or eight with two waves, which
  // issue twice the copies each).
  constexpr int KRMAX = NWAVE == 2 ? 8 : 4;
  constexpr int KREG = G::KPW < KRMAX ? G::KPW : KRMAX;
  constexpr int KPK = (KREG + 1) / 2;
  uint32_t koff2[KPK];
#pragma unroll
  for (int i2 = 0; i2 < KPK; ++i2) {
    uint32_t pk = k_offset(2 * i2);
    if (2 * i2 + 1 < KREG) pk |= k_offset(2 * i2 + 1) << 16;
    koff2[i2] = pk;
  }
  static_assert(BT * D * 2 <= 0x8000, "K copy offsets fit in 15 bits");
  // V copy j (j = wave + NWAVE i): physical chunk p of row r holds logical
  // chunk p with its segment bits XOR-ed by vx(r).  Copy i covers the rows of
  // copy 0 plus 64 NWAVE / NCH * i, whose vx is the same, so its offsets are
  // those of copy 0 plus VSTRIDE i bytes (a wave-uniform soffset).
  uint32_t voff0;
  {
    const int slot = 64 * wave + lane;
    const int row = slot / G::NCH;
    const int p = slot % G::NCH;
    const int ch = (((p >> 2) ^ vx<D>(row)) << 2) | (p & 3);
    voff0 = static_cast<uint32_t>((row * D + ch * 8) * 2);
  }
  constexpr uint32_t VSTRIDE = (64 * NWAVE / G::NCH) * D * 2;
  static_assert(VSTRIDE == 1024 * NWAVE, "V copy stride");
  const int kinst = (G::KINS - wave + NWAVE - 1) / NWAVE;   // K copies issued
  // Every wave issues at least KINS / NWAVE of them: stated so that those
  // copies need no branch.
  auto has_k_copy = [&](int i) {
    return i < G::KINS / NWAVE || i < kinst;
  };

  const int ntiles = MK ? ntl : (kv_end + BT - 1) / BT;
  const int nblk = 2 * ntiles;          // key blocks of BC keys
  // Steps 1 .. nsteps run in rounds of four; step b ends with O += P(b-1)
  // V(b-1), so the last real block is done at step nblk.  Blocks past the
  // real ones are virtual: their copies read zeros (the buffer descriptors
  // end at kv_end) and their scores are masked, so their p are 0.
  const int nsteps = (nblk + 3) & ~3;

  // Descriptors of the K / V rows [kv0, kv_end) of this (batch, KV head):
  // copies of rows past the last key this workgroup needs read zeros.
  auto rsrc_at = [&](const uint16_t* base, int kv0) {
    const int rows = max(kv_end - kv0, 0);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base + static_cast<int64_t>(kv0) * D), 0,
        rows * D * 2, 0x00020000);
  };
  // PS: tiles past this unit's last key are the next unit's first tiles
  // (same N, so kv0 - kv_end is their first key).
  // The next unit's K and V (null when there is none), formed once.
  const uint16_t* nkp = nullptr;
  const uint16_t* nvp = nullptr;
  if constexpr (PS) {
    const uint16_t* nq;
    if (!next_unit(nq, nkp, nvp)) nkp = nvp = nullptr;
  }
  auto rsrc_kv = [&](const uint16_t* base, bool is_v, int kv0) {
    if (PS && nkp != nullptr && kv0 >= kv_end)
      return rsrc_at(is_v ? nvp : nkp, kv0 - kv_end);
    return rsrc_at(base, kv0);
  };
  auto copy_k = [&](int tile, const uint4* stage) {
    const auto rs = rsrc_at(kp, tkv(tile));
#pragma unroll
    for (int i = 0; i < G::KPW; ++i)
      if (has_k_copy(i))
        copy_to_lds(rs, stage + 64 * (wave + NWAVE * i),
                    i < KREG ? (koff2[i >> 1] >> (16 * (i & 1))) & 0xFFFFu
                             : k_offset(i));
  };
  auto copy_v = [&](int tile, const uint4* stage) {
    const auto rs = rsrc_at(vp, tkv(tile));
#pragma unroll
    for (int i = 0; i < G::VPW; ++i)
      copy_to_lds(rs, stage + 64 * (wave + NWAVE * i), voff0, VSTRIDE * i);
  };
  // Copy n of the NCOPY copies a wave issues per tile pair: V copies first,
  // then K copies (the last K window only on the waves that have one).
  constexpr int NCOPY = G::VPW + G::KPW;
  auto copy_nth = [&](int n, __amdgpu_buffer_rsrc_t rk,
                      __amdgpu_buffer_rsrc_t rv, const uint4* kw,
                      const uint4* vw) {
    if (n < G::VPW) {
      copy_to_lds(rv, vw + 64 * (wave + NWAVE * n), voff0, VSTRIDE * n);
    } else {
      const int i = n - G::VPW;
      if (has_k_copy(i))
        copy_to_lds(rk, kw + 64 * (wave + NWAVE * i),
                    i < KREG ? (koff2[i >> 1] >> (16 * (i & 1))) & 0xFFFFu
                             : k_offset(i));
    }
  };

  // ---- per-lane LDS read offsets (bytes) ----
  //   K (A operand of S^T): row sigma(li) of the 32-key half kh of a stage,
  //   chunk h * NCH/2 + s.
  const int rd_k = (sigma(li) * G::KSL + h * (G::NCH / 2)) * 16;
  //   V (transposing read): lane 16 g + 4 R + j reads key row
  //   32 kh + 16 u + 8 h + 4 t4 + R at d = 32 db + 16 (g % 2) + 8 (j & 1)
  //   + 4 (j >> 1); the output lane then holds 4 keys of
  //   d = 32 db + sigma(lane % 32).  The 64-byte segment index sits in
  //   address bits 6-7 (bit 6 for D = 64) and is the only part that depends
  //   on db: rd_v0 ^ (db << 6).
  const int tr_R = (lane >> 2) & 3;
  const int tr_j = lane & 3;
  int rd_v0;
  {
    const int r = 8 * h + tr_R;
    const int seg = vx<D>(r);                        // segment of db = 0
    const int ch = 4 * seg + 2 * ((lane >> 4) & 1) + (tr_j & 1);
    rd_v0 = (r * G::NCH + ch) * 16 + 8 * (tr_j >> 1);
  }

  // ---- running softmax state (per lane and query block; halves agree) ----
  f32x16_t oacc[NQB][G::NDB];
  float m_run[NQB];
  float l_run[NQB];                     // this lane's half of the row sums
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
#pragma unroll
    for (int i = 0; i < G::NDB; ++i) oacc[j][i] = f32x16_t{};
    m_run[j] = -__builtin_inff();
    l_run[j] = 0.f;
  }
  const float c = a.c;

  // Hide the scores of keys a row may not see (causal: key > query;
  // ragged tail: key >= N) by setting them to -inf.  Lane half h holds keys
  // kv0 + 16 (r / 8) + 8 h + (r % 8) of the 32-key block.
  // VL: vis[j] says whether the row of query block j sees any key of the
  // block (rows that have seen none so far must take the exact step on the
  // first block where they do).
  // MK: mwv[j] holds the mask word of the block for this lane's row of
  // query block j (bits past NK cleared).
  uint32_t mwv[NQB];
  auto apply_mask = [&](f32x16_t (&s)[NQB], int kv0, bool (&vis)[NQB]) {
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      const int qrow = qw0 + 32 * j + li;
      if constexpr (MK) {
        // Lane half h holds keys 8 h + kx, kx = 16 (r / 8) + r % 8.
        const uint32_t mb = mwv[j] >> (8 * h);
        vis[j] = (mb & 0x00FF00FFu) != 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kx = 16 * (r >> 3) + (r & 7);
          if (!((mb >> kx) & 1u)) s[j][r] = -__builtin_inff();
        }
      } else if constexpr (VL) {
        // This row's visible keys [jlo, jhi], relative to the lane's first
        // key of the block: score r (key base + kx) is kept iff
        // rlo <= kx <= rhi.
        const int base = kv_begin + kv0 + 8 * h;
        const int jlo = wl < 0 ? 0 : qrow + off - wl;
        const int jhi = wr < 0 ? NK - 1 : min(NK - 1, qrow + off + wr);
        const int rlo = jlo - base, rhi = jhi - base;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kx = 16 * (r >> 3) + (r & 7);
          if (!(kx >= rlo && kx <= rhi)) s[j][r] = -__builtin_inff();
        }
        // The lane's keys are kx in 0..7 and 16..23.
        vis[j] = rlo <= rhi && ((rlo <= 7 && rhi >= 0) ||
                                (rlo <= 23 && rhi >= 16));
      } else if constexpr (CAUSAL) {
        // Score r holds key kvl + kx with kx = 16 (r / 8) + r % 8 and kvl
        // this lane's first key of the block: causal hides kx > qrow - kvl
        // (one compare with a constant per score); keys past NK occur in
        // the last block only (a uniform branch).
        const int kvl = kv0 + 8 * h;
        const int lim = qrow - kvl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kx = 16 * (r >> 3) + (r & 7);
          if (kx > lim) s[j][r] = -__builtin_inff();
        }
        if (kv0 + BC > NK) {
          const int lim_n = NK - 1 - kvl;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kx = 16 * (r >> 3) + (r & 7);
            if (kx > lim_n) s[j][r] = -__builtin_inff();
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 16 * (r >> 3) + 8 * h + (r & 7);
          if (key >= NK) s[j][r] = -__builtin_inff();
        }
      }
    }
  };
  auto masked_at = [&](int blk) {
    const int kv0 = kv_begin + blk * BC;
    if constexpr (VL)
      return (kv0 + BC > NK) || (wr >= 0 && kv0 + BC - 1 > qw0 + off + wr) ||
             (wl >= 0 && kv0 < qw0 + QPW - 1 + off - wl);
    else
      return (kv0 + BC > NK) || (CAUSAL && kv0 + BC - 1 > qw0);
  };
  // MK: the mask words of block blk (tile position blk / 2, half blk % 2)
  // for this lane's rows, bits past NK cleared; a virtual block's are 0.
  // MK: the mask words of the rows of this lane for two tiles in flight:
  // mt[slot][j][half] for tile position p in slot p % 2, bits past NK
  // cleared (a virtual tile's are 0).  A tile's words are fetched with its
  // K copy, two steps before the first block of the tile is masked.
  uint32_t mt[2][NQB][2];
  uint32_t mtk[2][2];                     // per slot and half: bits < NK
  auto fetch_mask_tile = [&](int kvt, bool full, uint32_t (&d)[NQB][2],
                             uint32_t (&dk)[2]) {
    // The words are only combined with their keep masks when used, so the
    // loads stay in flight; a tile every row sees whole needs none, and a
    // virtual tile keeps nothing.
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int kvb = kvt + BC * hb;
      const int kin = NK - kvb;
      dk[hb] = kin >= 32 ? ~0u : (kin > 0 ? (1u << kin) - 1u : 0u);
    }
    if (full) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int j = 0; j < NQB; ++j) d[j][hb] = ~0u;
    } else {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int wi = min((kvt + BC * hb) >> 5, a.mw - 1);
#pragma unroll
        for (int j = 0; j < NQB; ++j) d[j][hb] = mrow[j][wi];
      }
    }
  };
  // Whether block blk needs the mask applied: MK, unless every lane's rows
  // see all of its keys (a wave-uniform test on the loaded words).
  auto block_masked = [&](int blk) {
    if constexpr (MK) {
      bool full = true;
#pragma unroll
      for (int j = 0; j < NQB; ++j) full = full && mwv[j] == ~0u;
      return __builtin_amdgcn_ballot_w64(!full) != 0;
    } else {
      return masked_at(blk);
    }
  };

  // Exact step for a block whose P (formed with the held m) has a lane sum
  // above 2^TAU, or inf / NaN: from the block's scores s, move each query
  // block's m to its row maximum if that is larger, rescale O and l, and
  // form P again in w.  Returns the new lane sums in ls.
  auto exact_block = [&](const f32x16_t (&s)[NQB], uint32_t (&w)[8 * NQB],
                         float (&ls)[NQB]) {
    acc_read_fence();
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      float mx = s[j][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
      mx = half_max(mx);
      const float m_blk = (mx == -__builtin_inff()) ? mx : mx * c;
      const float m_new = fmaxf(m_run[j], m_blk);
      const float alpha = (m_new == -__builtin_inff())
                              ? 1.0f
                              : __builtin_amdgcn_exp2f(m_run[j] - m_new);
      m_run[j] = m_new;
      l_run[j] *= alpha;
      // One accumulator at a time (16 vector registers of temporaries).
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[j][db][r] *= alpha;
      }
      __builtin_amdgcn_sched_barrier(0);
      // A row with no visible key so far keeps m = -inf; its p are all 0.
      const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[j][2 * q], c, -m_use));
        const float p1 =
            __builtin_amdgcn_exp2f(fmaf(s[j][2 * q + 1], c, -m_use));
        w[8 * j + q] = pack_bf16x2(p0, p1);
        sum += p0 + p1;
      }
      ls[j] = sum;
    }
    acc_write_fence();
  };

  // K fragment s (k-step over d) of the 32-key half kh of stage ks.
  auto kfrag = [&](const uint4* ks, int kh, int s) {
    const uint8_t* p = reinterpret_cast<const uint8_t*>(ks) + rd_k +
                       32 * kh * G::KSL * 16 + 16 * s;
    return *reinterpret_cast<const uint4*>(p);
  };
  // Transposed V fragment f = (db, u) (two 8-byte reads, hf = 0, 1) of the
  // 32-key half kh of stage vs: d block db, 16-key step u.
  auto vread = [&](const uint4* vs, int kh, int f, int hf) {
    const int db = f % G::NDB;
    const int u = f / G::NDB;
    const uint8_t* p = reinterpret_cast<const uint8_t*>(vs) +
                       (rd_v0 ^ (db << 6)) +
                       (32 * kh + 16 * u + 4 * hf) * G::NCH * 16;
    return lds_read_tr16(p);
  };

  constexpr int NQK = NQB * G::NKS;     // scores MFMAs per step
  constexpr int NPV = 2 * NQB * G::NDB; // P V MFMAs per step
  static_assert(NQK == NPV, "one scores MFMA per P V MFMA");
  constexpr int NSL = NQK;              // issue slots per step
  constexpr int NPR = 8 * NQB;          // score pairs per lane per step
  constexpr int PPS = NPR / NSL;        // score pairs turned into P per slot
  constexpr int KPF = 2;                // K fragments read ahead
  constexpr int VPF = 2;                // V fragments read ahead
  constexpr int NVF = 2 * G::NDB;       // V fragments per step

  // tmax (MK): the largest tile position the next step looks up, if that
  // is a copy step (else -1).
  auto wait_copies_and_sync = [&](int tmax) {
    if constexpr (MK) {
      if (tmax >= 0) advance_list(tmax);
      // The 2 NQB mask-word loads issued after the last tile copies may
      // stay in flight (memory loads complete in order).
      static_assert(2 * NQB <= 15, "vmcnt field");
      __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * NQB));
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt: any
    }
    __syncthreads();
  };

  auto mfma_pv = [&](const i16x4_t (&vv)[2], const bf16x8_t& pb,
                     f32x16_t& acc) {
    const bf16x8_t v8 = __builtin_bit_cast(
        bf16x8_t,
        __builtin_shufflevector(vv[0], vv[1], 0, 1, 2, 3, 4, 5, 6, 7));
    mfma_pv_acc(v8, pb, acc);
  };

  // Copies of a SYNC step: CPS per issue slot from slot 1 on (NCS slots),
  // then (MK) the mask words of K's new tile.
  constexpr int CPS = (NCOPY + NSL - 3) / (NSL - 2);
  constexpr int NCS = (NCOPY + CPS - 1) / CPS;
  static_assert(NCS + 2 <= NSL, "copies and mask words fit the issue slots");
  static_assert(G::NKS - KPF == NVF - VPF,
                "K and V read-ahead cross into the next step in one slot");
  // Step blk of the three-stage pipeline.  On entry `s` holds the (masked)
  // scores of block blk and `pp` the settled P of block blk-1.  The K stage
  // kr (32-key half KH) holds block blk+1, the V stage vr (half VH) block
  // blk-1.  Every issue slot pairs one MFMA of the scores of block blk+1
  // (QK) and one MFMA of O += P(blk-1) V(blk-1) (PV) with PPS score pairs
  // of block blk turned into P (p = exp2(S c - m), fp32 lane sums, bf16
  // pack).  Masked scores are -inf and give p = 0 (the launcher keeps
  // c > 0).  A SYNC step (odd blk) starts the copies of tiles (blk-1)/2 + 2
  // (K, into kw) and (blk-1)/2 + 1 (V, into vw).
  // K and V fragments are read KPF / VPF fragments ahead of their MFMA, and
  // the read-ahead runs on into the next step (stages krn / vrn, halves
  // KHN / VHN), so a step starts with its first operands in registers: on
  // entry kf / vf hold this step's first KPF / VPF fragments.  When the
  // next step is a SYNC step, its stages were just filled by copies, and
  // the stages this step reads are the ones the next step's copies
  // overwrite: before the first read of the next stage, every wave waits
  // for its own reads and copies and meets the others at the barrier.
  // VL: whether the block now in `s` holds a key each row sees.
  bool svis[NQB];
  auto step = [&](int blk, f32x16_t (&s)[NQB], bf16x8_t (&pp)[NQB][2],
                  uint4 (&kf)[KPF], i16x4_t (&vf)[VPF][2],
                  const uint4* kr, const uint4* vr, const uint4* kw,
                  const uint4* vw, const uint4* krn, const uint4* vrn,
                  auto kh_tag, auto vh_tag, auto khn_tag, auto vhn_tag,
                  auto sync_tag, auto pv_tag, auto nsync_tag, auto ms_tag) {
    constexpr int KH = decltype(kh_tag)::value;
    constexpr int MS = decltype(ms_tag)::value;   // MK: mask-word slot
    constexpr int VH = decltype(vh_tag)::value;
    constexpr int KHN = decltype(khn_tag)::value;
    constexpr int VHN = decltype(vhn_tag)::value;
    constexpr bool SYNC = decltype(sync_tag)::value;
    constexpr bool QK = true;
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr bool NSYNC = decltype(nsync_tag)::value;
    // Two query blocks: consecutive products share operand A (the two
    // scores products of a K fragment in even slots, the two P V products
    // of a V fragment in odd slots) instead of alternating scores and P V
    // products; measured 1.1-1.8% faster (same GPU, bit-identical).
    constexpr bool PAIRED = NQB == 2 && PV && QK;
    // One query block (32-row waves: the variable-length and masked
    // configurations): even slots issue the scores products of two
    // consecutive K fragments, odd slots the P V products of two
    // consecutive V fragments (which share operand B, P of the same 16
    // keys); measured 0.6-2.3% faster on those launches, bit-identical.
    constexpr bool PAIR1 = FA_PAIR1 != 0 && NQB == 1 && PV && QK;
    // SYNC steps start the copies of tiles (blk-1)/2 + 2 (K, into kw) and
    // (blk-1)/2 + 1 (V, into vw), one per issue slot from slot 1 on, so
    // that their issue overlaps the matrix work; their descriptors are
    // formed after the first MFMA has been issued.
    const int tile = (blk - 1) >> 1;
    __amdgpu_buffer_rsrc_t rk, rv;
    int kvk = 0;                        // MK: first key of K's new tile
    bool fullk = true;                  // MK: every row sees it whole
    // MK: mask words of block blk+1 (masked at the end of this step).
    // MK: the mask words of block blk+1 (tile slot MS, half KH).
    if constexpr (MK) {
#pragma unroll
      for (int j = 0; j < NQB; ++j) mwv[j] = mt[MS][j][KH] & mtk[MS][KH];
    }
    float mu[NQB];
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      // VL: a row that has seen no key yet (m = -inf) forms P against 0, so
      // that fully masked blocks give p = 0 instead of NaN; the first block
      // in which it sees a key takes the exact step (sum test below), which
      // sets m from that block.
      if constexpr (VM)
        mu[j] = (m_run[j] == -__builtin_inff()) ? 0.f : m_run[j];
      else
        mu[j] = m_run[j];
    }
    f32x16_t sn[NQB];
#pragma unroll
    for (int j = 0; j < NQB; ++j) sn[j] = f32x16_t{};
    uint32_t w[NPR];
    // Lane sums of the even / odd pairs of each query block, started by its
    // first two pairs (8 j and 8 j + 1).
    float lse_[NQB], lso_[NQB];
    uint4 kcur = {}, kcur2 = {};
    i16x4_t vcur[2] = {}, vcur2[2] = {};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      // Each slot: an MFMA, then p = exp2(S c - m) for PPS pairs while it
      // runs; a second MFMA, then the bf16 packs and lane sums of those
      // pairs while that one runs.  With one wave per SIMD, this keeps
      // vector work under both MFMAs and puts the exp latency between the
      // two halves.  The two MFMAs are a scores and a P V product, or
      // (PAIRED) the two scores products of a K fragment (even slots) or
      // the two P V products of a V fragment (odd slots), or (PAIR1) two
      // scores products (even slots) or two P V products (odd slots) of
      // consecutive fragments.
      if constexpr (PAIR1) {
        const int f = i & ~1;             // first of the slot's two fragments
        if (i % 2 == 0) {
          kcur = kf[0];
          kcur2 = kf[1];
          if (f + 2 < G::NKS) {
            kf[0] = kfrag(kr, KH, f + 2);
            kf[1] = kfrag(kr, KH, f + 3);
          } else {
            // First reads of the next step's stage; every read of this
            // step's stages is issued.
            if (NSYNC) wait_copies_and_sync(blk / 2 + 2);
            kf[0] = kfrag(krn, KHN, 0);
            kf[1] = kfrag(krn, KHN, 1);
          }
          sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(kcur), qf[0][f], sn[0], 0, 0, 0);
        } else {
          vcur[0] = vf[0][0];
          vcur[1] = vf[0][1];
          vcur2[0] = vf[1][0];
          vcur2[1] = vf[1][1];
          if (f + 2 < NVF) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              vf[t][0] = vread(vr, VH, f + 2 + t, 0);
              vf[t][1] = vread(vr, VH, f + 2 + t, 1);
            }
          } else {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              vf[t][0] = vread(vrn, VHN, t, 0);
              vf[t][1] = vread(vrn, VHN, t, 1);
            }
          }
          mfma_pv(vcur, pp[0][f / G::NDB], oacc[0][f % G::NDB]);
        }
      }
      if constexpr (PAIRED) {
        // Odd slot: first P V product of V fragment i / 2 (query block 0),
        // with that fragment's read-ahead replaced (this step's stage, or
        // the next step's, whose barrier came in slot NSL - 4).
        if (i % 2 == 1) {
          const int f = i / 2;
          vcur[0] = vf[f % VPF][0];
          vcur[1] = vf[f % VPF][1];
          if (f + VPF < NVF) {
            vf[f % VPF][0] = vread(vr, VH, f + VPF, 0);
            vf[f % VPF][1] = vread(vr, VH, f + VPF, 1);
          } else {
            vf[f % VPF][0] = vread(vrn, VHN, f + VPF - NVF, 0);
            vf[f % VPF][1] = vread(vrn, VHN, f + VPF - NVF, 1);
          }
          mfma_pv(vcur, pp[0][f / G::NDB], oacc[0][f % G::NDB]);
        }
      }
      if (QK && !PAIR1 && (!PAIRED || i % 2 == 0)) {
        // k-step i / NQB for query block i % NQB: the fragment serves all
        // (PAIRED: k-step i / 2, query block 0; block 1 follows below).
        const int f = i / NQB, qb = PAIRED ? 0 : i % NQB;
        if (qb == 0) {
          kcur = kf[f % KPF];
          if (f + KPF < G::NKS) kf[f % KPF] = kfrag(kr, KH, f + KPF);
        }
        sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(kcur), qf[qb][f], sn[qb], 0, 0, 0);
        if (qb == 0 && f + KPF >= G::NKS) {
          // First read of the next step's stage (V's follows in this slot).
          // The next step (blk + 1) is a copy step: it looks up tile
          // positions blk / 2 + 1 and blk / 2 + 2.
          if (NSYNC && f + KPF == G::NKS) wait_copies_and_sync(blk / 2 + 2);
          kf[f % KPF] = kfrag(krn, KHN, f + KPF - G::NKS);
        }
      }
      if constexpr (SYNC) {
        if (i == 0) {
          if constexpr (MK) {
            kvk = tkv(tile + 2);
            fullk = tfull(tile + 2);
            rk = rsrc_at(kp, kvk);
            rv = rsrc_kv(vp, true, tkv(tile + 1));
          } else {
            rk = rsrc_kv(kp, false, tkv(tile + 2));
            rv = rsrc_kv(vp, true, tkv(tile + 1));
          }
        }
        if constexpr (SERIAL_COPIES) {
          if (i == 1) wait_copies_and_sync(-1);
        }
        if (i >= 1 && i <= NCS) {
#pragma unroll
          for (int c = 0; c < CPS; ++c)
            if ((i - 1) * CPS + c < NCOPY)
              copy_nth((i - 1) * CPS + c, rk, rv, kw, vw);
        }
        if constexpr (SERIAL_COPIES) {
          if (i == NCS) wait_copies_and_sync(-1);
        }
        // MK: the mask words of K's tile, after its copies.
        if constexpr (MK) {
          if (i == NCS + 1)
            fetch_mask_tile(kvk, fullk, mt[1 - MS], mtk[1 - MS]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // VL (two waves per SIMD): a wave in its exponentials, packs and sums
      // issues before the other one; measured 0.7-1.3% faster than equal
      // priorities (and within noise on the masked configuration).
      if constexpr (VL) __builtin_amdgcn_s_setprio(1);
      float e[PPS][2];
#pragma unroll
      for (int q = 0; q < PPS; ++q) {
        const int pr = i * PPS + q;                 // pair 0 .. NPR-1
        const int j = pr >> 3, r = 2 * (pr & 7);    // query block, register
        e[q][0] = __builtin_amdgcn_exp2f(fmaf(s[j][r], c, -mu[j]));
        e[q][1] = __builtin_amdgcn_exp2f(fmaf(s[j][r + 1], c, -mu[j]));
        // Pin the work to this slot (otherwise it is sunk towards its use,
        // past the scheduling fences).
        asm volatile("" : "+v"(e[q][0]), "+v"(e[q][1]));
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (PAIR1) {
        const int f = i & ~1;
        if (i % 2 == 0)
          sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(kcur2), qf[0][f + 1], sn[0], 0, 0, 0);
        else
          mfma_pv(vcur2, pp[0][(f + 1) / G::NDB], oacc[0][(f + 1) % G::NDB]);
      } else if constexpr (PAIRED) {
        // Second product of the slot: the same operand A as the first.
        const int f = i / 2;
        if (i % 2 == 0)
          sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(kcur), qf[1][f], sn[1], 0, 0, 0);
        else
          mfma_pv(vcur, pp[1][f / G::NDB], oacc[1][f % G::NDB]);
      } else if constexpr (PV) {
        // V fragment i / NQB = (db, u) for query block i % NQB.
        const int f = i / NQB, qb = i % NQB;
        if (qb == 0) {
          vcur[0] = vf[f % VPF][0];
          vcur[1] = vf[f % VPF][1];
          if (f + VPF < NVF) {
            vf[f % VPF][0] = vread(vr, VH, f + VPF, 0);
            vf[f % VPF][1] = vread(vr, VH, f + VPF, 1);
          }
        }
        mfma_pv(vcur, pp[qb][f / G::NDB], oacc[qb][f % G::NDB]);
      }
      if constexpr (!PAIRED && !PAIR1) {
        // Read-ahead into the next step, which always has a P V product
        // (after the barrier above when the next step is a SYNC step).
        const int f = i / NQB, qb = i % NQB;
        if (qb == 0 && f + VPF >= NVF) {
          vf[f % VPF][0] = vread(vrn, VHN, f + VPF - NVF, 0);
          vf[f % VPF][1] = vread(vrn, VHN, f + VPF - NVF, 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < PPS; ++q) {
        const int pr = i * PPS + q;
        const int j = pr >> 3;
        const float p0 = e[q][0], p1 = e[q][1];
        w[pr] = pack_bf16x2(p0, p1);
        float& acc = (pr & 1) ? lso_[j] : lse_[j];
        if (pr < 8 * j + 2)
          acc = p0 + p1;
        else
          acc += p0 + p1;
        asm volatile("" : "+v"(w[pr]), "+v"(acc));
      }
      if constexpr (VL) __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Accept P of block blk or take the exact step first, then add it to l.
    float ls[NQB];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < NQB; ++j) {
      ls[j] = lse_[j] + lso_[j];
      bad = bad || !(ls[j] <= TAU_EXP2);
      if constexpr (VM)
        bad = bad || (m_run[j] == -__builtin_inff() && svis[j]);
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(bad) != 0, 0))
      exact_block(s, w, ls);  // rare
#pragma unroll
    for (int j = 0; j < NQB; ++j) l_run[j] += ls[j];
#pragma unroll
    for (int j = 0; j < NQB; ++j)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        pp[j][u] = __builtin_bit_cast(
            bf16x8_t,
            make_uint4(w[8 * j + 4 * u], w[8 * j + 4 * u + 1],
                       w[8 * j + 4 * u + 2], w[8 * j + 4 * u + 3]));
    if constexpr (QK) {
      bool vn[NQB];
#pragma unroll
      for (int j = 0; j < NQB; ++j) vn[j] = true;
      if (__builtin_expect(block_masked(blk + 1), 0))
        apply_mask(sn, (blk + 1) * BC, vn);
#pragma unroll
      for (int j = 0; j < NQB; ++j) s[j] = sn[j];
      if constexpr (VM) {
#pragma unroll
        for (int j = 0; j < NQB; ++j) svis[j] = vn[j];
      }
    }
  };

  // ---- prologue: K tiles 0 and 1, V tile 0 into LDS; scores of block 0 --
  // Stages: tile t lives in Ks[t % 2] / Vs[t % 2].  Step blk reads K block
  // blk+1 (tile (blk+1)/2, half (blk+1)%2) and V block blk-1; SYNC steps
  // are the odd ones.  With period 4 in blk:
  //   blk%4 == 0: K Ks0 half 1, V Vs1 half 1
  //   blk%4 == 1: K Ks1 half 0, V Vs0 half 0, SYNC: fill Vs1, Ks0
  //   blk%4 == 2: K Ks1 half 1, V Vs0 half 1
  //   blk%4 == 3: K Ks0 half 0, V Vs1 half 0, SYNC: fill Vs0, Ks1
  if (!have) {
    copy_k(0, Ks0);
    copy_v(0, Vs0);
    copy_k(1, Ks1);
  }
  settle_q();
  wait_copies_and_sync(-1);
  f32x16_t s[NQB];
#pragma unroll
  for (int j = 0; j < NQB; ++j) s[j] = f32x16_t{};
#pragma unroll
  for (int i = 0; i < NQK; ++i)
    s[i % NQB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        as_bf16x8(kfrag(Ks0, 0, i / NQB)), qf[i % NQB][i / NQB], s[i % NQB],
        0, 0, 0);
#pragma unroll
  for (int j = 0; j < NQB; ++j) svis[j] = true;
  if constexpr (MK) {
    // Tiles 0 and 1 into slots 0 and 1; block 0 is tile 0, half 0.
    fetch_mask_tile(tkv(0), tfull(0), mt[0], mtk[0]);
    fetch_mask_tile(tkv(1), tfull(1), mt[1], mtk[1]);
#pragma unroll
    for (int j = 0; j < NQB; ++j) mwv[j] = mt[0][j][0] & mtk[0][0];
  }
  if (block_masked(0)) apply_mask(s, 0, svis);
  // Reference max from block 0 (without VL every row sees key 0, so m is
  // finite for the rows that exist; with VL a row may see nothing yet and
  // keep m = -inf).
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    float mx = s[j][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
    mx = half_max(mx);
    m_run[j] = (mx == -__builtin_inff()) ? mx : mx * c;
  }
  bf16x8_t pp[NQB][2];

  using T0 = Tag<false>;
  using T1 = Tag<true>;
  // ---- step 0 (no P V yet), then rounds of four steps ----
  // Step 0's first K fragments (block 1: stage Ks0, half 1); it has no
  // P V product, so its V read-ahead only serves step 1.
  uint4 kf[KPF];
  i16x4_t vf[VPF][2] = {};
#pragma unroll
  for (int i = 0; i < KPF; ++i) kf[i] = kfrag(Ks0, 1, i);
  // Arguments: K / V stages read, K / V stages written (SYNC steps), the
  // next step's K / V stages, halves read now and next, SYNC, P V, next
  // step SYNC, mask-word slot of the block masked at the end of the step.
  step(0, s, pp, kf, vf, Ks0, Vs1, Ks0, Vs0, Ks1, Vs0, Int<1>{}, Int<1>{},
       Int<0>{}, Int<0>{}, T0{}, T0{}, T1{}, Int<0>{});
  for (int blk = 1; blk <= nsteps; blk += 4) {
    step(blk, s, pp, kf, vf, Ks1, Vs0, Ks0, Vs1, Ks1, Vs0, Int<0>{},
         Int<0>{}, Int<1>{}, Int<1>{}, T1{}, T1{}, T0{}, Int<1>{});
    step(blk + 1, s, pp, kf, vf, Ks1, Vs0, Ks0, Vs1, Ks0, Vs1, Int<1>{},
         Int<1>{}, Int<0>{}, Int<0>{}, T0{}, T1{}, T1{}, Int<1>{});
    step(blk + 2, s, pp, kf, vf, Ks0, Vs1, Ks1, Vs0, Ks0, Vs1, Int<0>{},
         Int<0>{}, Int<1>{}, Int<1>{}, T1{}, T1{}, T0{}, Int<0>{});
    step(blk + 3, s, pp, kf, vf, Ks0, Vs1, Ks1, Vs0, Ks1, Vs0, Int<1>{},
         Int<1>{}, Int<0>{}, Int<0>{}, T0{}, T1{}, T1{}, Int<0>{});
  }

  // PS: the next unit's first tiles are in the stages (the last step waited
  // for every copy); its Q loads go out before this unit's epilogue.
  have = false;
  if constexpr (PS) {
    const uint16_t *nq, *nk, *nv;
    if (next_unit(nq, nk, nv)) {
      load_q(nq, wave * QPW, BR);
      have = true;
    } else {
#pragma unroll
      for (int j = 0; j < NQB; ++j)
#pragma unroll
        for (int t = 0; t < G::NKS; ++t) qraw[j][t] = make_uint4(0, 0, 0, 0);
    }
  }

  // PS: the output offsets are formed here, not held across the loop.
  if constexpr (PS) asm volatile("" : "+s"(qrow0));
  // ---- epilogue: O / l in bf16 (RNE), LSE in natural log ----
  acc_read_fence();
#pragma unroll
  for (int j = 0; j < NQB; ++j) {
    const int qrow = qw0 + 32 * j + li;
    const float l_tot = half_sum(l_run[j]);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qrow < NQ) {
      uint16_t* op = static_cast<uint16_t*>(a.o) + (qrow0 + qrow) * D;
      // Accumulator row m <-> d = 32 db + sigma(m): lane half h holds
      // d = 32 db + 16 u + 8 h + (0..7) in registers 8 u .. 8 u + 7.
#pragma unroll
      for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x16_t& o = oacc[j][db];
          uint4 w;
          w.x = pack_bf16x2(o[8 * u + 0] * inv, o[8 * u + 1] * inv);
          w.y = pack_bf16x2(o[8 * u + 2] * inv, o[8 * u + 3] * inv);
          w.z = pack_bf16x2(o[8 * u + 4] * inv, o[8 * u + 5] * inv);
          w.w = pack_bf16x2(o[8 * u + 6] * inv, o[8 * u + 7] * inv);
          *reinterpret_cast<uint4*>(op + 32 * db + 16 * u + 8 * h) = w;
        }
      }
      if (h == 0) {
        const float m_fin = (m_run[j] == -__builtin_inff()) ? 0.f : m_run[j];
        float* lp = a.lse + qrow0 + qrow;
        *lp = (l_tot > 0.f) ? (m_fin + __log2f(l_tot)) * 0.69314718055994531f
                            : -__builtin_inff();
      }
    }
  }
  }  // units
}

}  // namespace

// Compute units of the current device (0 if it cannot be read), read once
// per device.
static int cu_count() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount,
                              dev) == hipSuccess)
      cached[dev] = n;
  }
  return cached[dev];
}

// 64 rows per wave, one wave per SIMD (halves LDS reads per FLOP against
// 32-row waves; the single wave per SIMD is issue-bound but still ahead):
// measured 4-5% ahead non-causal, 0.4-1.9% causal.
template <int D, bool CAUSAL>
static hipError_t launch(const FwdArgs& a, int grid, hipStream_t stream) {
  constexpr int NQB = 2;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, NQB>), dim3(grid),
                     dim3(Waves<NQB>::NTHR), 0, stream, a);
  return hipGetLastError();
}

// Variable-length batches and sliding windows (d = 128): the causal
// template with 8 waves of 32 rows, per-sequence offsets and window
// masks.  a.nqb covers the longest query sequence.
hipError_t launch_fwd_varlen_bf16(FwdArgs a, int max_q, hipStream_t stream) {
  constexpr int BR = Waves<1>::BR;
  a.nqb = static_cast<int>((static_cast<long long>(max_q) + BR - 1) / BR);
  const long long grid = static_cast<long long>(a.B) * a.H * a.nqb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  if (static_cast<long long>(a.total_k) * 128 * 2 > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  a.xcd_chunk = a.Hkv % 8 == 0;
  hipLaunchKernelGGL((fwd_bf16_kernel<128, true, 1, true>), dim3((int)grid),
                     dim3(Waves<1>::NTHR), 0, stream, a);
  return hipGetLastError();
}

// Forward under an arbitrary visibility bit mask (d = 128): the non-causal
// configuration over the listed key tiles with per-block mask words.
// a.total_q / a.total_k are Nq / Nk.
hipError_t launch_fwd_masked_bf16(FwdArgs a, hipStream_t stream) {
  // 128 query rows per workgroup, so that a workgroup streams the tiles its
  // own 128 rows see (not the union over 256), as four waves of 32 rows:
  // two workgroups per CU (LDS) give two waves per SIMD.  Measured against
  // two waves of 64 rows (one per SIMD) on B4 H16 N8192: block-sparse
  // 0.507 -> 0.470 ms, all-visible 2.047 -> 1.981, causal-shaped 1.194 ->
  // 1.128, 50% random 2.454 -> 2.289.
  using W = Waves<1, 4>;
  a.nqb = static_cast<int>((static_cast<long long>(a.total_q) + W::BR - 1) /
                           W::BR);
  const long long grid = static_cast<long long>(a.B) * a.H * a.nqb;
  if (grid > 0x7FFFFFFFLL || a.total_k > MASK_MAX_NK)
    return hipErrorInvalidConfiguration;
  if (static_cast<long long>(a.total_k) * 128 * 2 > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  a.mw = (a.total_k + 31) / 32;
  a.xcd_chunk = grid % 8 == 0;
  hipLaunchKernelGGL((fwd_bf16_kernel<128, false, 1, false, true, 4>),
                     dim3((int)grid), dim3(W::NTHR), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(FwdArgs a, int d, bool causal, hipStream_t stream) {
  constexpr int BR = Waves<2>::BR;
  a.nqb = static_cast<int>((static_cast<long long>(a.N) + BR - 1) / BR);
  const long long grid = static_cast<long long>(a.B) * a.H * a.nqb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  // Per-(batch, KV head) byte ranges are addressed by 32-bit buffer
  // offsets.
  if (static_cast<long long>(a.N) * d * 2 > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  const int bh = a.B * a.H;
  a.xcd_chunk = causal ? (bh % 8 == 0) : (grid % 8 == 0);
  // Persistent launch (one workgroup per CU looping over the units): dense
  // non-causal, every unit whole (N a multiple of BR), more units than CUs,
  // and a CU count that keeps each workgroup on one XCD's units.
  int g = static_cast<int>(grid);
  a.persist = 0;
  if (FA_PERSIST && !causal && a.N % BR == 0) {
    const int ncu = cu_count();
    if (ncu > 0 && ncu % 8 == 0 && ncu < grid) {
      a.persist = 1;
      g = ncu;
    }
  }
  if (d == 64) {
    return causal ? launch<64, true>(a, g, stream)
                  : launch<64, false>(a, g, stream);
  }
  return causal ? launch<128, true>(a, g, stream)
                : launch<128, false>(a, g, stream);
}

}  // namespace fa
