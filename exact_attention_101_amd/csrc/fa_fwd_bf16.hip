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
//   * workgroup = 4 waves, BR = 128 query rows (32 per wave), K/V blocks of
//     BC = 64 keys.  K and V blocks go from HBM/L2 straight into LDS with
//     buffer_load_dwordx4 ... lds (no register staging), into four distinct
//     LDS stage arrays (two for K, two for V) so the compiler can tell the
//     in-flight copies from the stages being read;
//   * scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16: the accumulator column is the query, so each
//     lane holds 32 scores of one query and the row max / row sum are
//     in-lane plus one v_permlane32_swap between the two lane halves;
//   * Q lives in registers as the B operand for the whole kernel; the
//     contraction over d is permuted so that lane half h holds the
//     contiguous d-range [h*D/2, (h+1)*D/2);
//   * K rows are loaded in sigma order (fa_common.h), so the fp32 score
//     accumulator, converted to bf16, is directly the B operand of
//     O^T = V^T P^T; V stays in its [key][d] layout in LDS and the A operand
//     (V^T) is read with the transposing ds_read_b64_tr_b16;
//   * softmax in fp32 registers in the log2 domain: p = exp2(S*c - m) with
//     c = |scale| * log2(e) (one FMA + v_exp_f32 per score), fp32 row sums;
//   * the two matrix products overlap the softmax inside each wave (the
//     intra-group overlap of the FlashAttention-3 summary, section
//     «Assincronia: sobreposição de GEMM e Softmax»): while the matrix core
//     computes the scores of block t+1, the vector unit turns the scores of
//     block t into P; then the P V product of block t runs.  The order is
//     pinned with scheduling-group barriers;
//   * the running maximum m is a reference value, not necessarily the exact
//     maximum: any m gives the same softmax (the shift cancels between
//     numerator and denominator), so P is first formed with the m already
//     held.  Only if a lane's sum of the block's p exceeds 2^TAU (some score
//     rose more than TAU log2 units above m; also inf / NaN, which is how the
//     first block, with m = -inf, is caught) does the wave take the exact
//     step: row maximum of the block, move m, rescale O and l, form P
//     again.  All p stay in [0, 2^TAU], and the common path computes no row
//     maximum at all;
//   * LDS layouts are chosen so every MFMA operand read is free of bank
//     conflicts: K rows are padded by one 16-byte slot, V rows XOR their
//     64-byte segments with the key's position in its group of 4.
#include "fa_common.h"

namespace fa {

namespace {

constexpr int BR = 128;
constexpr int BC = 64;
constexpr int NTHR = 256;
constexpr float TAU_EXP2 = 256.0f;   // 2^TAU, TAU = 8 (log2 units)

typedef __attribute__((ext_vector_type(4))) short i16x4_t;

template <bool V>
struct Tag {
  static constexpr bool value = V;
};

template <int D>
struct Geo {
  static constexpr int NCH = D / 8;                // 16-byte chunks per row
  static constexpr int NDB = D / 32;               // 32-wide d blocks
  static constexpr int NKS = D / 16;               // QK^T MFMA k-steps
  // K: rows padded to NCH + 1 slots (16 bytes each): 16 consecutive rows at
  // the same chunk land in 16 different 4-bank groups.
  static constexpr int KSL = NCH + 1;
  static constexpr int KSLOTS = BC * KSL;
  static constexpr int KINS = KSLOTS / 64;         // 64-lane copies per block
  static constexpr int KPW = (KINS + 3) / 4;       // per wave (at most)
  // V: unpadded rows, 64-byte segments XOR-swizzled.
  static constexpr int VSLOTS = BC * NCH;
  static constexpr int VINS = VSLOTS / 64;
  static constexpr int VPW = VINS / 4;
  static_assert(KSLOTS % 64 == 0 && VSLOTS % 256 == 0, "copy tiling");
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

// Instruction-order groups for the scheduler.
#define SCHED_GROUP(mask, n, id) __builtin_amdgcn_sched_group_barrier(mask, n, id)
constexpr int SG_VALU = 0x002 | 0x400;   // VALU incl. transcendental
constexpr int SG_MFMA = 0x008;
constexpr int SG_DSR = 0x100;

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NTHR, 2)
fwd_bf16_kernel(const FwdArgs a) {
  using G = Geo<D>;
  __shared__ uint4 Ks0[G::KSLOTS];
  __shared__ uint4 Ks1[G::KSLOTS];
  __shared__ uint4 Vs0[G::VSLOTS];
  __shared__ uint4 Vs1[G::VSLOTS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int li = lane & 31;             // MFMA column / row-in-block
  const int h = lane >> 5;              // lane half

  int bh, qb;
  map_work(blockIdx.x, gridDim.x, a.B * a.H, a.nqb, CAUSAL, a.xcd_chunk, bh,
           qb);
  const int b = bh / a.H;
  const int hq = bh % a.H;
  const int hk = hq / a.group;
  const int N = a.N;
  const int q0 = qb * BR;
  const int qw0 = q0 + wave * 32;       // first query row of this wave
  const int qrow = qw0 + li;            // this lane's query row

  const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                       (static_cast<int64_t>(b) * a.H + hq) * N * D;
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) +
                       (static_cast<int64_t>(b) * a.Hkv + hk) * N * D;
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) +
                       (static_cast<int64_t>(b) * a.Hkv + hk) * N * D;

  // ---- Q -> registers (B operand of S^T = K Q^T) ----
  bf16x8_t qf[G::NKS];
  {
    const uint32_t flip = a.neg ? 0x80008000u : 0u;
    const bool ok = qrow < N;
    const uint16_t* src = qp + static_cast<int64_t>(ok ? qrow : N - 1) * D +
                          h * (D / 2);
#pragma unroll
    for (int s = 0; s < G::NKS; ++s) {
      uint4 u = keep_if(ldg16(src + 8 * s), ok);
      u.x ^= flip; u.y ^= flip; u.z ^= flip; u.w ^= flip;
      qf[s] = as_bf16x8(u);
    }
  }

  // ---- per-lane byte offsets of this wave's block copies ----
  // K copy j (j = wave + 4 i) fills slots 64 j .. 64 j + 63: lane L writes
  // slot 64 j + L = row * KSL + chunk; pad slots re-read the last chunk.
  // Offsets are below 2^15: copies 2 i2 and 2 i2 + 1 share a register, and
  // a copy past the first four (the last window, one wave) computes its
  // offsets when issued.
  auto k_offset = [&](int i) {
    const int slot = 64 * (wave + 4 * i) + lane;
    const int row = slot / G::KSL;
    const int ch = min(slot - row * G::KSL, G::NCH - 1);
    return static_cast<uint32_t>((row * D + ch * 8) * 2);
  };
  constexpr int KREG = G::KPW < 4 ? G::KPW : 4;   // copies with a register
  constexpr int KPK = (KREG + 1) / 2;
  uint32_t koff2[KPK];
#pragma unroll
  for (int i2 = 0; i2 < KPK; ++i2) {
    uint32_t pk = k_offset(2 * i2);
    if (2 * i2 + 1 < KREG) pk |= k_offset(2 * i2 + 1) << 16;
    koff2[i2] = pk;
  }
  static_assert(BC * D * 2 <= 0x8000, "K copy offsets fit in 15 bits");
  // V copy j (j = wave + 4 i): physical chunk p of row r holds logical chunk
  // p with its segment bits XOR-ed by vx(r).  Copy i covers the rows of copy
  // 0 plus 256 / NCH * i, whose vx is the same, so its offsets are those of
  // copy 0 plus 4096 i bytes (a wave-uniform soffset).
  uint32_t voff0;
  {
    const int slot = 64 * wave + lane;
    const int row = slot / G::NCH;
    const int p = slot % G::NCH;
    const int ch = (((p >> 2) ^ vx<D>(row)) << 2) | (p & 3);
    voff0 = static_cast<uint32_t>((row * D + ch * 8) * 2);
  }
  static_assert((256 / G::NCH) * D * 2 == 4096, "V copy stride");
  const int kinst = (G::KINS - wave + 3) / 4;   // copies this wave issues

  // Descriptors of the K / V rows [kv0, N) of this (batch, KV head): copies
  // of rows past N read zeros.
  auto rsrc_at = [&](const uint16_t* base, int kv0) {
    const int rows = max(N - kv0, 0);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base + static_cast<int64_t>(kv0) * D), 0,
        rows * D * 2, 0x00020000);
  };
  auto copy_k = [&](int t, const uint4* stage) {
    const auto rs = rsrc_at(kp, t * BC);
#pragma unroll
    for (int i = 0; i < G::KPW; ++i)
      if (i < kinst)
        copy_to_lds(rs, stage + 64 * (wave + 4 * i),
                    i < KREG ? (koff2[i >> 1] >> (16 * (i & 1))) & 0xFFFFu
                             : k_offset(i));
  };
  auto copy_v = [&](int t, const uint4* stage) {
    const auto rs = rsrc_at(vp, t * BC);
#pragma unroll
    for (int i = 0; i < G::VPW; ++i)
      copy_to_lds(rs, stage + 64 * (wave + 4 * i), voff0, 4096u * i);
  };

  // ---- per-lane LDS read offsets (bytes) ----
  //   K (A operand of S^T): row sigma(li) + 32 kb, chunk h * NCH/2 + s.
  const int rd_k = (sigma(li) * G::KSL + h * (G::NCH / 2)) * 16;
  //   V (transposing read): lane 16 g + 4 R + j reads key row
  //   32 kb + 16 u + 8 h + 4 t4 + R at d = 32 db + 16 (g % 2) + 8 (j & 1)
  //   + 4 (j >> 1); the output lane then holds 4 keys of
  //   d = 32 db + sigma(lane % 32).
  const int tr_R = (lane >> 2) & 3;
  const int tr_j = lane & 3;
  //   The 64-byte segment index sits in address bits 6-7 (bit 6 for D = 64)
  //   and is the only part that depends on db: rd_v0 ^ (db << 6).
  int rd_v0;
  {
    const int r = 8 * h + tr_R;
    const int seg = vx<D>(r);                        // segment of db = 0
    const int ch = 4 * seg + 2 * ((lane >> 4) & 1) + (tr_j & 1);
    rd_v0 = (r * G::NCH + ch) * 16 + 8 * (tr_j >> 1);
  }

  // ---- running softmax state (per lane = per query; both halves agree) ----
  f32x16_t oacc[G::NDB];
#pragma unroll
  for (int i = 0; i < G::NDB; ++i) oacc[i] = f32x16_t{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;                    // this lane's half of the row sum
  const float c = a.c;

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;

  // Hide the scores of keys a row may not see (causal: key > query;
  // ragged tail: key >= N) by setting them to -inf.  Lane half h holds keys
  // kv0 + 32 kb + 16 (r / 8) + 8 h + (r % 8).
  auto apply_mask = [&](f32x16_t (&s)[2], int kv0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + 32 * kb + 16 * (r >> 3) + 8 * h + (r & 7);
        const bool ok = key < N && (!CAUSAL || key <= qrow);
        if (!ok) s[kb][r] = -__builtin_inff();
      }
    }
  };
  auto masked_at = [&](int t) {
    const int kv0 = t * BC;
    return (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0);
  };

  // Exact step for a block whose P (formed with the held m) has a lane sum
  // above 2^TAU, or inf / NaN: from the block's scores sx, move m to the
  // row maximum if that is larger, rescale O and l, and form P again in w.
  // Returns the new lane sum of the block.
  auto exact_block = [&](const f32x16_t (&sx)[2], uint32_t (&w)[16]) {
    float mx = sx[0][0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = fmaxf(mx, sx[i >> 4][i & 15]);
    mx = half_max(mx);
    const float m_tile = (mx == -__builtin_inff()) ? mx : mx * c;
    const float m_new = fmaxf(m_run, m_tile);
    const float alpha = (m_new == -__builtin_inff())
                            ? 1.0f
                            : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < G::NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    // A row with no visible key so far keeps m = -inf; its p are all 0.
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    float ls = 0.f;
#pragma unroll
    for (int pr = 0; pr < 16; ++pr) {
      const int kb = pr >> 3, r = 2 * (pr & 7);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sx[kb][r], c, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sx[kb][r + 1], c, -m_use));
      w[pr] = pack_bf16x2(p0, p1);
      ls += p0 + p1;
    }
    return ls;
  };
  // K fragment i of the scores product: k-step s = i / 2, key block
  // kb = i % 2 (alternating the two accumulators).
  auto kfrag = [&](const uint4* ks, int i) {
    const uint8_t* p = reinterpret_cast<const uint8_t*>(ks) + rd_k +
                       32 * (i & 1) * G::KSL * 16 + 16 * (i >> 1);
    return *reinterpret_cast<const uint4*>(p);
  };
  // Transposed V fragment j (two 8-byte reads) of P V step i = (kb, u, db).
  auto vread = [&](const uint4* vs, int i, int half) {
    const int db = i % G::NDB;
    const int u = (i / G::NDB) & 1;
    const int kb = i / (2 * G::NDB);
    const uint8_t* p = reinterpret_cast<const uint8_t*>(vs) + (rd_v0 ^ (db << 6)) +
                       (32 * kb + 16 * u + 4 * half) * G::NCH * 16;
    return lds_read_tr16(p);
  };

  constexpr int NQK = 2 * G::NKS;       // MFMAs of the scores product
  constexpr int NPV = 4 * G::NDB;       // MFMAs of the P V product
  static_assert(NQK == NPV, "one scores MFMA per P V MFMA");
  constexpr int NSL = NQK;              // issue slots per step
  constexpr int PPS = 16 / NSL;         // score pairs turned into P per slot
  constexpr int KPF = 2;                // K fragments read ahead
  constexpr int VPF = 2;                // V steps read ahead

  auto pack_p = [&](const uint32_t (&w)[16], bf16x8_t (&pb)[2][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        pb[kb][u] = __builtin_bit_cast(
            bf16x8_t, make_uint4(w[8 * kb + 4 * u], w[8 * kb + 4 * u + 1],
                                 w[8 * kb + 4 * u + 2], w[8 * kb + 4 * u + 3]));
  };

  // Accept P of block t (scores s, P packed in w, lane sum ls) or take the
  // exact step first, then add the block to l.
  auto settle = [&](const f32x16_t (&s)[2], uint32_t (&w)[16], float ls) {
    const bool bad = !(ls <= TAU_EXP2);
    if (__builtin_amdgcn_ballot_w64(bad) != 0) ls = exact_block(s, w);  // rare
    l_run += ls;
  };

  auto wait_copies_and_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt: any
    __syncthreads();
  };

  // Step t of the three-stage pipeline.  On entry `s` holds the (masked)
  // scores of block t and `pp` the settled P of block t-1; the K stage kr
  // holds block t+1 and the V stage vr block t-1.  Every issue slot pairs
  // one MFMA of the scores of block t+1 (QK) and one MFMA of
  // O += P(t-1) V(t-1) (PV) with PPS score pairs of block t turned into P
  // (p = exp2(S c - m), fp32 lane sum, bf16 pack), so the vector unit works
  // while the matrix core runs.  Masked scores are -inf and give p = 0 (the
  // launcher keeps c > 0); with m = -inf every p is inf or NaN, which the
  // sum test sends to the exact step.  The step first waits for the copies
  // of the previous step and then starts those of V(t) into vw and K(t+2)
  // into kw.
  auto step = [&](int t, f32x16_t (&s)[2], bf16x8_t (&pp)[2][2],
                  const uint4* kr, const uint4* vr, const uint4* kw,
                  const uint4* vw, auto qk_tag, auto pv_tag) {
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr bool PV = decltype(pv_tag)::value;
    wait_copies_and_sync();
    copy_v(t, vw);
    if (t + 2 < ntiles) copy_k(t + 2, kw);
    const float m_use = m_run;
    uint4 kf[KPF];
    i16x4_t vf[VPF][2];
    if constexpr (QK) {
#pragma unroll
      for (int i = 0; i < KPF; ++i) kf[i] = kfrag(kr, i);
    }
    if constexpr (PV) {
#pragma unroll
      for (int i = 0; i < VPF; ++i) {
        vf[i][0] = vread(vr, i, 0);
        vf[i][1] = vread(vr, i, 1);
      }
    }
    f32x16_t sn[2];
    sn[0] = f32x16_t{};
    sn[1] = f32x16_t{};
    uint32_t w[16];
    float ls0 = 0.f, ls1 = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NSL; ++i) {
      if constexpr (QK) {
        const uint4 kk = kf[i % KPF];
        if (i + KPF < NQK) kf[i % KPF] = kfrag(kr, i + KPF);
        sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(kk), qf[i >> 1], sn[i & 1], 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < PPS; ++q) {
        const int pr = i * PPS + q;                 // pair 0..15
        const int kb = pr >> 3, r = 2 * (pr & 7);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -m_use));
        const float p1 =
            __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], c, -m_use));
        w[pr] = pack_bf16x2(p0, p1);
        if (pr & 1) ls1 += p0 + p1; else ls0 += p0 + p1;
        // Pin the work to this slot (otherwise it is sunk towards its use
        // in the next step, past the scheduling fences).
        asm volatile("" : "+v"(w[pr]), "+v"(ls0), "+v"(ls1));
      }
      if constexpr (PV) {
        const i16x4_t lo = vf[i % VPF][0], hi = vf[i % VPF][1];
        if (i + VPF < NPV) {
          vf[i % VPF][0] = vread(vr, i + VPF, 0);
          vf[i % VPF][1] = vread(vr, i + VPF, 1);
        }
        const int db = i % G::NDB;
        const int u = (i / G::NDB) & 1;
        const int kb = i / (2 * G::NDB);
        const bf16x8_t vv = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pp[kb][u],
                                                           oacc[db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    settle(s, w, ls0 + ls1);
    bf16x8_t pb[2][2];
    pack_p(w, pb);
    if constexpr (QK) {
      if (masked_at(t + 1)) apply_mask(sn, (t + 1) * BC);
      s[0] = sn[0];
      s[1] = sn[1];
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int u = 0; u < 2; ++u) pp[kb][u] = pb[kb][u];
  };

  // Last product: O += P(T-1) V(T-1) from the V stage vr (k-slot (h, e) of
  // each 16-key step is key 32 kb + 16 u + 8 h + e on both operands).
  auto final_pv = [&](const uint4* vr, const bf16x8_t (&pp)[2][2]) {
    wait_copies_and_sync();
    i16x4_t vf[VPF][2];
#pragma unroll
    for (int i = 0; i < VPF; ++i) {
      vf[i][0] = vread(vr, i, 0);
      vf[i][1] = vread(vr, i, 1);
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      const i16x4_t lo = vf[i % VPF][0], hi = vf[i % VPF][1];
      if (i + VPF < NPV) {
        vf[i % VPF][0] = vread(vr, i + VPF, 0);
        vf[i % VPF][1] = vread(vr, i + VPF, 1);
      }
      const int db = i % G::NDB;
      const int u = (i / G::NDB) & 1;
      const int kb = i / (2 * G::NDB);
      const bf16x8_t vv = __builtin_bit_cast(
          bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pp[kb][u],
                                                         oacc[db], 0, 0, 0);
    }
  };

  // ---- prologue: K blocks 0 and 1 into LDS, scores of block 0 ----
  // Stages by parity of the step t: step t reads K(t+1) from Ks[(t+1) % 2]
  // and V(t-1) from Vs[(t-1) % 2] and fills Ks[t % 2] with K(t+2) and
  // Vs[t % 2] with V(t).
  copy_k(0, Ks0);
  if (ntiles > 1) copy_k(1, Ks1);
  wait_copies_and_sync();
  f32x16_t s[2];
  s[0] = f32x16_t{};
  s[1] = f32x16_t{};
#pragma unroll
  for (int i = 0; i < NQK; ++i)
    s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        as_bf16x8(kfrag(Ks0, i)), qf[i >> 1], s[i & 1], 0, 0, 0);
  if (masked_at(0)) apply_mask(s, 0);
  {
    // Reference max from block 0 (every row sees key 0, so m is finite).
    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = fmaxf(mx, s[i >> 4][i & 15]);
    mx = half_max(mx);
    m_run = (mx == -__builtin_inff()) ? mx : mx * c;
  }
  bf16x8_t pp[2][2];

  // ---- steps 0 .. T-1, then the last product ----
  const int last = ntiles - 1;
  if (last == 0) {
    step(0, s, pp, Ks1, Vs1, Ks0, Vs0, Tag<false>{}, Tag<false>{});
    final_pv(Vs0, pp);
  } else {
    step(0, s, pp, Ks1, Vs1, Ks0, Vs0, Tag<true>{}, Tag<false>{});
    int t = 1;
    for (; t + 2 <= last; t += 2) {            // steps t (odd), t + 1 (even)
      step(t, s, pp, Ks0, Vs0, Ks1, Vs1, Tag<true>{}, Tag<true>{});
      step(t + 1, s, pp, Ks1, Vs1, Ks0, Vs0, Tag<true>{}, Tag<true>{});
    }
    if (t < last) {                           // one more odd step
      step(t, s, pp, Ks0, Vs0, Ks1, Vs1, Tag<true>{}, Tag<true>{});
      ++t;
    }
    if (t & 1) {                              // t == last
      step(t, s, pp, Ks0, Vs0, Ks1, Vs1, Tag<false>{}, Tag<true>{});
      final_pv(Vs1, pp);
    } else {
      step(t, s, pp, Ks1, Vs1, Ks0, Vs0, Tag<false>{}, Tag<true>{});
      final_pv(Vs0, pp);
    }
  }

  // ---- epilogue: O / l in bf16 (RNE), LSE in natural log ----
  const float l_tot = half_sum(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* op = static_cast<uint16_t*>(a.o) +
                   ((static_cast<int64_t>(b) * a.H + hq) * N + qrow) * D;
    // Accumulator row m <-> d = 32 db + sigma(m): lane half h holds
    // d = 32 db + 16 u + 8 h + (0..7) in registers 8 u .. 8 u + 7.
#pragma unroll
    for (int db = 0; db < G::NDB; ++db) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint4 w;
        w.x = pack_bf16x2(oacc[db][8 * u + 0] * inv, oacc[db][8 * u + 1] * inv);
        w.y = pack_bf16x2(oacc[db][8 * u + 2] * inv, oacc[db][8 * u + 3] * inv);
        w.z = pack_bf16x2(oacc[db][8 * u + 4] * inv, oacc[db][8 * u + 5] * inv);
        w.w = pack_bf16x2(oacc[db][8 * u + 6] * inv, oacc[db][8 * u + 7] * inv);
        *reinterpret_cast<uint4*>(op + 32 * db + 16 * u + 8 * h) = w;
      }
    }
    if (h == 0) {
      const float m_fin = (m_run == -__builtin_inff()) ? 0.f : m_run;
      float* lp = a.lse + (static_cast<int64_t>(b) * a.H + hq) * N + qrow;
      *lp = (l_tot > 0.f) ? (m_fin + __log2f(l_tot)) * 0.69314718055994531f
                          : -__builtin_inff();
    }
  }
}

}  // namespace

template <int D, bool CAUSAL>
static hipError_t launch(const FwdArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(grid), dim3(NTHR), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(FwdArgs a, int d, bool causal, hipStream_t stream) {
  a.nqb = (a.N + BR - 1) / BR;
  const long long grid = static_cast<long long>(a.B) * a.H * a.nqb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  // Per-(batch, KV head) byte ranges are addressed by 32-bit buffer
  // offsets.
  if (static_cast<long long>(a.N) * d * 2 > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  const int bh = a.B * a.H;
  a.xcd_chunk = causal ? (bh % 8 == 0) : (grid % 8 == 0);
  if (d == 64) {
    return causal ? launch<64, true>(a, (int)grid, stream)
                  : launch<64, false>(a, (int)grid, stream);
  }
  return causal ? launch<128, true>(a, (int)grid, stream)
                : launch<128, false>(a, (int)grid, stream);
}

}  // namespace fa
