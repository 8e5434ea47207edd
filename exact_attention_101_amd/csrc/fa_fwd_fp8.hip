// FP8 (OCP e4m3) FlashAttention forward for gfx950 (MI355X), d = 128.
//
// Same tiling and online softmax as the bf16 kernel (FlashAttention v1 post,
// DeepSchool #630, sections «Тайлинг (Tiling)» and «Онлайн-Softmax»), with
// both products on the FP8 matrix cores, the low-precision path of the
// FlashAttention-3 summary (GeekNews), sections «Principais tecnologias do
// FlashAttention-3» and «Novos recursos de hardware da GPU Hopper».
//
//   * Inputs are e4m3 codes with per-tensor descales dQ, dK, dV read from
//     device memory (no host synchronisation).  The score scale folds in
//     dQ * dK; dV multiplies the output in the epilogue.
//   * S^T = K Q^T and O^T = V^T P^T run on v_mfma_scale_f32_32x32x64_f8f6f4
//     with neutral (2^0) block scales, fp32 accumulation.  Each lane owns
//     one query; the lane's 32 scores of a 64-key tile, rounded to e4m3, are
//     exactly its 32-byte B operand of the P V product (K rows in sigma
//     order, fa_common.h), and the V^T operand comes from the transposing
//     ds_read_b64_tr_b8.
//   * Workgroup = 4 waves of 32 query rows (BR = 128), two workgroups per
//     CU, so two waves per SIMD: with fp8 the matrix work per score halves,
//     so the vector work of the softmax needs the issue slots of two waves,
//     and waves of different workgroups never wait at each other's barrier.
//     K and V tiles of 64 keys go from HBM/L2 straight into LDS with
//     buffer_load_dwordx4 ... lds (two 1 KB windows of each per wave),
//     double-buffered.
//   * A three-stage software pipeline runs in every step t: one issue slot
//     per MFMA pair, the scores MFMA of tile t+1, p = exp2(S c - m + 8) for
//     four score pairs of tile t, the P V MFMA of tile t-1, then the e4m3
//     packs and lane sums of those pairs (the intra-group overlap of the
//     FlashAttention-3 summary, section «Assincronia»).
//   * P is stored as p * 2^8 in e4m3 (keeps small weights out of the
//     subnormal range), which must stay at most 448.  O and l are kept
//     relative to a per-row base m0 (block 0's row maximum) and are never
//     rescaled: tile t forms p against m0 + E_t, where E_t is the smallest
//     integer (never decreasing) that keeps the tile's row maximum within
//     log2(448/256) of it, and the P V MFMA takes the per-lane block scale
//     2^E_t of the f8f6f4 instruction, so O accumulates p * 2^8 * 2^E_t
//     relative to m0 exactly.  Two row sums follow it: lq over the e4m3
//     values the product used, from one more MFMA per tile with an all-ones
//     A operand and the same block scale (O = acc / lq, so a row whose
//     weight sits on one key is not off by that key's rounding, up to 2^-4),
//     and l, the lanes' fp32 sums of p before rounding times 2^E_t (the
//     LSE).  Both carry the same 2^8, which cancels in O and is removed from
//     the LSE.  Only if E passes 64 (scores rising more than 64
//     log2 units above block 0) are O and l renormalised, to keep fp32
//     headroom.
#include "fa_common.h"

namespace fa {

namespace {

constexpr int D = 128;
constexpr int BT = 64;               // keys per tile (= per step)
// Waves per workgroup.  Two workgroups share a CU (registers and LDS allow
// it), so each SIMD runs two waves that never wait on each other's barrier.
constexpr int NWAVE_FP8 = 4;
constexpr int NCH = D / 16;          // 16-byte chunks per row (8)
constexpr float P_SHIFT = 8.0f;      // P is stored as p * 2^8
// p * 2^8 <= 448 (largest finite e4m3) when the score is at most
// log2(448 / 256) = 0.807 log2 units above the reference.
constexpr float P_HEADROOM = 0.8f;
constexpr int E_RENORM = 64;         // renormalise O, l beyond this shift

typedef __attribute__((ext_vector_type(2))) int i32x2_t;

template <bool V>
struct Tag {
  static constexpr bool value = V;
};

// K tile [key][d] bytes: physical 16-byte chunk of (row r, chunk c).  The
// reading lane i uses row r = sigma(i) (+32 kb), so the XOR term depends on
// the lane only and 16 lanes reading the same logical chunk hit 16
// different 4-bank groups.
__device__ __forceinline__ int kswz(int r, int c) {
  const int t = sigma(r & 31);
  return c ^ ((t & 7) ^ ((t >> 3) & 1));
}

// V tile [key][d] bytes: the 8 key rows of one transposing read differ in
// (r % 2, (r >> 1) % 4); XOR-ing the 32-byte segment with (r >> 1) % 4
// spreads them over all banks.
__device__ __forceinline__ int vswz(int r, int c) {
  return c ^ (2 * ((r >> 1) & 3));
}

// Transposing 8-bit LDS read: in each group of 16 lanes, lanes 2R and 2R+1
// supply 8 consecutive bytes each (row R = 16 bytes), and output lane i gets
// byte i of rows R = 0..7.
__device__ __forceinline__ i32x2_t lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2_t*)(p));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 values to e4m3 (RNE, saturating) into the low (hi = 0) or high
// (hi = 1) 16 bits of `old`.
__device__ __forceinline__ int pack_fp8x2(float a, float b, int old, int hi) {
  return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
            : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

// Maximum that propagates NaN (IEEE maximum): unlike fmaxf it needs no
// quieting of its inputs, and three-input forms fold into v_maximum3_f32.
__device__ __forceinline__ float maxf(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return maxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16_t mfma_f8(const i32x8_t& a,
                                            const i32x8_t& b,
                                            const f32x16_t& c) {
  // cbsz = blgp = 0: both operands e4m3; scale exponents 127 = 2^0.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0,
                                                         127, 0, 127);
}
// Same with the B operand scaled by 2^(eb - 127) (E8M0 block scale, one per
// lane: each lane's 32 k-values of its column).
__device__ __forceinline__ f32x16_t mfma_f8_bscale(const i32x8_t& a,
                                                   const i32x8_t& b,
                                                   const f32x16_t& c,
                                                   int eb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0,
                                                         127, 0, eb);
}

// One 64-lane copy of 16 bytes per lane from `rsrc` (+ voffset bytes) into
// LDS at `dst` + 16 * lane.  Offsets past the descriptor's size read zeros.
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc,
                                            const uint4* dst,
                                            uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)(dst), 16, voffset, 0, 0,
      0);
}

template <bool CAUSAL, int NWAVE>
__global__ void __launch_bounds__(64 * NWAVE, 1)
fwd_fp8_kernel(const FwdArgs a) {
  constexpr int BR = 32 * NWAVE;               // query rows per workgroup
  // 1 KB copy windows per tile and operand, and how many each wave issues.
  constexpr int NWIN = BT * NCH / (64 * NWAVE);
  static_assert(NWIN * 64 * NWAVE == BT * NCH, "whole windows per wave");
  // Window w of wave v covers rows 8 (v + NWAVE w) .. +7: a multiple of 32
  // rows apart, so the swizzles (which depend on the row mod 32) repeat.
  static_assert(NWIN == 1 || (8 * NWAVE) % 32 == 0, "window spacing");
  constexpr uint32_t WIN_BYTES = 8 * NWAVE * D;  // global offset per window
  __shared__ uint4 Ks0[BT * NCH];
  __shared__ uint4 Ks1[BT * NCH];
  __shared__ uint4 Vs0[BT * NCH];
  __shared__ uint4 Vs1[BT * NCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int li = lane & 31;
  const int h = lane >> 5;

  int bh, qb;
  map_work(blockIdx.x, gridDim.x, a.B * a.H, a.nqb, CAUSAL, a.xcd_chunk, bh,
           qb);
  const int b = bh / a.H;
  const int hq = bh % a.H;
  const int hk = hq / a.group;
  const int N = a.N;
  const int q0 = qb * BR;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + li;

  float dq = 1.f, dk = 1.f, dv = 1.f;
  if (a.descale) {
    dq = a.descale[0];
    dk = a.descale[1];
    dv = a.descale[2];
  }
  // Scores enter exp2 as S * c with c = |scale| dQ dK log2(e); a negative
  // product is handled by negating Q's codes (sign bit) on load.  c is
  // floored so that a masked score (-inf) always gives p = 0.
  const float cs = a.scale * dq * dk * 1.4426950408889634f;
  const bool neg = cs < 0.f;
  const float c = fmaxf(fabsf(cs), 1e-30f);

  const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                      (static_cast<int64_t>(b) * a.H + hq) * N * D;
  const uint8_t* kp = static_cast<const uint8_t*>(a.k) +
                      (static_cast<int64_t>(b) * a.Hkv + hk) * N * D;
  const uint8_t* vp = static_cast<const uint8_t*>(a.v) +
                      (static_cast<int64_t>(b) * a.Hkv + hk) * N * D;

  // Q -> registers: k-step s covers d in [64 h + 32 s, +32) for lane half h.
  i32x8_t qf[2];
  {
    const uint32_t flip = neg ? 0x80808080u : 0u;
    const bool ok = qrow < N;
    const uint4* src = reinterpret_cast<const uint4*>(
        qp + static_cast<int64_t>(ok ? qrow : N - 1) * D + 64 * h);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4 u0 = keep_if(src[2 * s], ok);
      const uint4 u1 = keep_if(src[2 * s + 1], ok);
      qf[s] = i32x8_t{(int)(u0.x ^ flip), (int)(u0.y ^ flip),
                      (int)(u0.z ^ flip), (int)(u0.w ^ flip),
                      (int)(u1.x ^ flip), (int)(u1.y ^ flip),
                      (int)(u1.z ^ flip), (int)(u1.w ^ flip)};
    }
  }

  // ---- tile copies: wave w fills 64-slot window w of each stage ----
  // Lane L writes physical slot 64 w + L = row * NCH + physical chunk; the
  // logical chunk is recovered with the (involutive) swizzle.
  uint32_t koff, voff;
  {
    const int slot = 64 * wave + lane;
    const int r = slot / NCH, p = slot % NCH;
    koff = static_cast<uint32_t>(r * D + 16 * kswz(r, p));
    voff = static_cast<uint32_t>(r * D + 16 * vswz(r, p));
  }

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;   // last key needed + 1
  const int ntiles = (kv_end + BT - 1) / BT;
  // Steps 1 .. nsteps run in pairs; step t ends with O += P(t-1) V(t-1), so
  // the last real tile is done at step ntiles.  Tiles past the real ones
  // are virtual: their copies read zeros (the descriptors end at kv_end) and
  // their scores are masked, so their p are 0.
  const int nsteps = (ntiles + 1) & ~1;

  auto rsrc_at = [&](const uint8_t* base, int kv0) {
    const int rows = max(kv_end - kv0, 0);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(base + static_cast<int64_t>(kv0) * D), 0,
        rows * D, 0x00020000);
  };

  // ---- LDS read offsets ----
  //   K fragment (kb, s): row 32 kb + sigma(li), logical chunks 4 h + 2 s
  //   and 4 h + 2 s + 1.
  auto kfrag = [&](const uint4* ks, int kb, int s) {
    const int r = 32 * kb + sigma(li);
    const uint4* row = ks + r * NCH;
    const uint4 k0 = row[kswz(r, 4 * h + 2 * s)];
    const uint4 k1 = row[kswz(r, 4 * h + 2 * s + 1)];
    return i32x8_t{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w,
                   (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
  };
  //   Transposed V fragment of d block db: group g = lane / 16, lanes 2R + j
  //   of the group read key row 16 t8 + 8 h + R at bytes [32 db + 16 (g % 2)
  //   + 8 j, +8); output lane i then holds 8 keys of d = 32 db + 16 (g % 2)
  //   + i, for t8 = 0..3 (bytes 8 t8 .. 8 t8 + 7 of the A operand).
  const int tr_g = lane >> 4;
  const int tr_R = (lane >> 1) & 7;
  const int tr_j = lane & 1;
  const int tr_c = 2 * (tr_g & 1) + tr_j;        // 8-byte unit in a 32-d block
  auto vfrag = [&](const uint4* vs, int db) {
    int av[8];
#pragma unroll
    for (int t8 = 0; t8 < 4; ++t8) {
      const int r = 16 * t8 + 8 * h + tr_R;
      const int unit = 4 * db + tr_c;
      const uint8_t* p = reinterpret_cast<const uint8_t*>(
                             vs + r * NCH + vswz(r, unit >> 1)) +
                         8 * (unit & 1);
      const i32x2_t x = lds_read_tr8(p);
      av[2 * t8] = x[0];
      av[2 * t8 + 1] = x[1];
    }
    return i32x8_t{av[0], av[1], av[2], av[3], av[4], av[5], av[6], av[7]};
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16_t{};
  float m0 = 0.f;                       // per-row base, log2 units
  int e_cur = 0;                        // E of the tile whose P is formed
  float l_run = 0.f;                    // this lane's half of sum p*2^8*2^E
  // Row sums of the e4m3 P the product used, times 2^E, from a fifth MFMA
  // with an all-ones A: every row of the result is the column sum, so each
  // lane's element 0 is the sum for its own query.
  f32x16_t lacc = f32x16_t{};
  const int ONE4 = 0x38383838;          // four e4m3 1.0
  const i32x8_t ones = {ONE4, ONE4, ONE4, ONE4, ONE4, ONE4, ONE4, ONE4};

  // Lane half h holds keys kv0 + 32 kb + 16 (r / 8) + 8 h + (r % 8).
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
    const int kv0 = t * BT;
    return (kv0 + BT > N) || (CAUSAL && kv0 + BT - 1 > qw0);
  };

  // Row maximum of a tile's (masked) scores, both lane halves; -inf if
  // every key of the tile is hidden from the row.
  // A tree of three-input maxima: 32 values -> 12 -> 4 -> 1 in 16
  // v_maximum3_f32 (the maximum is exact, so the order is free).
  auto lane_max = [&](const f32x16_t (&s)[2]) {
    auto at = [&](int j) { return s[j >> 4][j & 15]; };
    float m1[12];
#pragma unroll
    for (int i = 0; i < 10; ++i)
      m1[i] = maxf(maxf(at(3 * i), at(3 * i + 1)), at(3 * i + 2));
    m1[10] = at(30);
    m1[11] = at(31);
    float m2[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m2[i] = maxf(maxf(m1[3 * i], m1[3 * i + 1]), m1[3 * i + 2]);
    return maxf(maxf(maxf(m2[0], m2[1]), m2[2]), m2[3]);
  };
  auto tile_max = [&](const f32x16_t (&s)[2]) {
    return half_max(lane_max(s));
  };
  // over(x): how many log2 units a raw score x lies above m0 + P_HEADROOM;
  // a tile's E must be at least over() of its row maximum.  Monotone in x
  // (c > 0), so a row's maximum passes E exactly when one of the row's two
  // lanes' maxima does.
  auto over = [&](float x) { return fmaf(x, c, -m0) - P_HEADROOM; };
  // E for a tile with row maximum mx (raw score): the smallest integer,
  // not below the previous one, with over(mx) <= E.
  auto next_e = [&](float mx, int e_prev) {
    if (mx == -__builtin_inff()) return e_prev;
    const float need = ceilf(over(mx));
    return need > static_cast<float>(e_prev) ? static_cast<int>(need)
                                              : e_prev;
  };

  auto wait_copies_and_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt: any
    __syncthreads();
  };

  // Step t of the three-stage pipeline.  On entry `s` holds the (masked)
  // scores of tile t and `pp` the settled P of tile t-1.  K stage kr holds
  // tile t+1, V stage vr tile t-1.  The step first waits for the copies of
  // the previous step, then starts those of tiles t+2 (K, into kw) and t
  // (V, into vw).  Slot i: scores MFMA i (key block i % 2, d step i / 2) of
  // tile t+1; p for pairs 4 i .. 4 i + 3 of tile t; P V MFMA of d block i
  // for tile t-1; e4m3 packs and lane sums of those pairs.
  auto step = [&](int t, f32x16_t (&s)[2], i32x8_t& pp, int& e_pp,
                  const uint4* kr, const uint4* vr, const uint4* kw,
                  const uint4* vw, auto pv_tag) {
    constexpr bool PV = decltype(pv_tag)::value;
    const auto rk = rsrc_at(kp, (t + 2) * BT);
    const auto rv = rsrc_at(vp, t * BT);
    wait_copies_and_sync();
    const float moff = P_SHIFT - (m0 + static_cast<float>(e_cur));
    const int eb = 127 + e_pp;          // 2^E of the P being multiplied
    i32x8_t kf = kfrag(kr, 0, 0);
    i32x8_t vf;
    if constexpr (PV) vf = vfrag(vr, 0);
    f32x16_t sn[2];
    sn[0] = f32x16_t{};
    sn[1] = f32x16_t{};
    // Packed P words: each is written as its low half, then its high half,
    // so its starting contents do not matter (left undefined, which spares
    // clearing them).  The lane sums start from the first two pairs.
    int pw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "=v"(pw[i]));
    float ls0, ls1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x8_t kcur = kf;
      if (i + 1 < 4) kf = kfrag(kr, (i + 1) & 1, (i + 1) >> 1);
      sn[i & 1] = mfma_f8(kcur, qf[i >> 1], sn[i & 1]);
      // Copies spread over the slots: V window i / 2 on even slots, K window
      // i / 2 on odd ones.
      if (i / 2 < NWIN) {
        const int w = i / 2;
        if (i % 2 == 0)
          copy_to_lds(rv, vw + 64 * (wave + NWAVE * w), voff + w * WIN_BYTES);
        else
          copy_to_lds(rk, kw + 64 * (wave + NWAVE * w), koff + w * WIN_BYTES);
      }
      __builtin_amdgcn_sched_barrier(0);
      float e[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pr = 4 * i + q;
        const int kb = pr >> 3, r = 2 * (pr & 7);
        e[q][0] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, moff));
        e[q][1] = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], c, moff));
        asm volatile("" : "+v"(e[q][0]), "+v"(e[q][1]));
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (PV) {
        const i32x8_t vcur = vf;
        if (i + 1 < 4) vf = vfrag(vr, i + 1);
        oacc[i] = mfma_f8_bscale(vcur, pp, oacc[i], eb);
        // Keeps the product in its slot: without a use here the compiler
        // sinks all four past the masking branch, after the exps.
        asm volatile("" : "+v"(oacc[i]));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int pr = 4 * i + q;
        pw[pr >> 1] = pack_fp8x2(e[q][0], e[q][1], pw[pr >> 1], pr & 1);
        float& ls = (q & 1) ? ls1 : ls0;
        if (pr < 2)
          ls = e[q][0] + e[q][1];
        else
          ls += e[q][0] + e[q][1];
        asm volatile("" : "+v"(pw[pr >> 1]), "+v"(ls));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // O is divided by the sum of the rounded values the P V product used,
    // so a row whose weight sits on one key still divides that key's value
    // by itself; l (fp32 p before rounding) gives the LSE.
    if constexpr (PV) lacc = mfma_f8_bscale(ones, pp, lacc, eb);
    l_run += __builtin_ldexpf(ls0 + ls1, e_cur);
    pp = i32x8_t{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
    e_pp = e_cur;
    if (masked_at(t + 1)) apply_mask(sn, (t + 1) * BT);
    s[0] = sn[0];
    s[1] = sn[1];
    // E changes only for a row whose maximum passes over() > E, which one
    // of the row's two lanes sees alone; the exchange between lane halves
    // and the update run only when some lane sees it (rare: E never falls).
    const float lmx = lane_max(s);
    if (__builtin_amdgcn_ballot_w64(over(lmx) > static_cast<float>(e_cur)) !=
        0) {
      e_cur = next_e(half_max(lmx), e_cur);
      if (__builtin_amdgcn_ballot_w64(e_cur > E_RENORM) != 0) {   // rare
        // Move the base up by E: O, l and the pending P's scale follow.
        const int sh = e_cur;
        const float f = __builtin_ldexpf(1.0f, -sh);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= f;
        l_run *= f;
#pragma unroll
        for (int r = 0; r < 16; ++r) lacc[r] *= f;
        m0 += static_cast<float>(sh);
        e_pp = max(e_pp - sh, -127);
        e_cur = 0;
      }
    }
  };

  // ---- prologue: K tiles 0 and 1 into LDS, scores of tile 0 ----
  // Stages: tile u lives in Ks[u % 2] / Vs[u % 2]; step t reads K(t+1) and
  // V(t-1), both from stage (t+1) % 2, and fills stage t % 2.
#pragma unroll
  for (int w = 0; w < NWIN; ++w) {
    copy_to_lds(rsrc_at(kp, 0), Ks0 + 64 * (wave + NWAVE * w),
                koff + w * WIN_BYTES);
    copy_to_lds(rsrc_at(kp, BT), Ks1 + 64 * (wave + NWAVE * w),
                koff + w * WIN_BYTES);
  }
  wait_copies_and_sync();
  f32x16_t s[2];
  s[0] = f32x16_t{};
  s[1] = f32x16_t{};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s[i & 1] = mfma_f8(kfrag(Ks0, i & 1, i >> 1), qf[i >> 1], s[i & 1]);
  if (masked_at(0)) apply_mask(s, 0);
  {
    // Base from tile 0 (every row sees key 0, so it is finite for the rows
    // that exist).
    const float mx = tile_max(s);
    m0 = (mx == -__builtin_inff()) ? 0.f : mx * c;
  }
  i32x8_t pp = {};
  int e_pp = 0;

  step(0, s, pp, e_pp, Ks1, Vs1, Ks0, Vs0, Tag<false>{});
  for (int t = 1; t <= nsteps; t += 2) {
    step(t, s, pp, e_pp, Ks0, Vs0, Ks1, Vs1, Tag<true>{});
    step(t + 1, s, pp, e_pp, Ks1, Vs1, Ks0, Vs0, Tag<true>{});
  }

  // Epilogue.  Accumulator row m <-> d = 32 db + m: lane half h holds runs
  // of 4 consecutive d at 32 db + 8 (r / 4) + 4 h.
  // O divides by the sum of the weights it was built from (the e4m3 values);
  // the LSE takes the sum of the unrounded p.
  const float l_tot = half_sum(l_run);
  const float lq_tot = lacc[0];
  const float inv = (lq_tot > 0.f) ? dv / lq_tot : 0.f;
  if (qrow < N) {
    uint16_t* op = static_cast<uint16_t*>(a.o) +
                   ((static_cast<int64_t>(b) * a.H + hq) * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 w;
        w.x = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        w.y = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * g + 4 * h) = w;
      }
    }
    if (h == 0) {
      float* lp = a.lse + (static_cast<int64_t>(b) * a.H + hq) * N + qrow;
      *lp = (l_tot > 0.f)
                ? (m0 + __log2f(l_tot) - P_SHIFT) * 0.69314718055994531f
                : -__builtin_inff();
    }
  }
}

}  // namespace

template <int NWAVE>
hipError_t launch_waves(FwdArgs a, bool causal, hipStream_t stream) {
  constexpr int BR = 32 * NWAVE;
  a.nqb = (a.N + BR - 1) / BR;
  const long long grid = static_cast<long long>(a.B) * a.H * a.nqb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  // Per-(batch, KV head) byte ranges are addressed by 32-bit buffer
  // offsets.
  if (static_cast<long long>(a.N) * D > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  const int bh = a.B * a.H;
  a.xcd_chunk = causal ? (bh % 8 == 0) : (grid % 8 == 0);
  if (causal) {
    hipLaunchKernelGGL((fwd_fp8_kernel<true, NWAVE>), dim3((int)grid),
                       dim3(64 * NWAVE), 0, stream, a);
  } else {
    hipLaunchKernelGGL((fwd_fp8_kernel<false, NWAVE>), dim3((int)grid),
                       dim3(64 * NWAVE), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(FwdArgs a, bool causal, hipStream_t stream) {
  return launch_waves<NWAVE_FP8>(a, causal, stream);
}

}  // namespace fa
