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
//   * S^T = K Q^T and O^T = V^T P^T run on v_mfma_scale_f32_32x32x64_f8f6f4,
//     fp32 accumulation.  Each lane owns one query; the lane's 32 scores of
//     a 64-key tile, rounded to e4m3, are exactly its 32-byte B operand of
//     the P V product (K rows in sigma order, fa_common.h), and the V^T
//     operand comes from the transposing ds_read_b64_tr_b8.
//   * P is stored as p * 2^8 in e4m3 (keeps small weights out of the
//     subnormal range), which must stay at most 448.  O and l are kept
//     relative to a per-row base m0 (tile 0's row maximum) and are never
//     rescaled: tile t forms p against m0 + E_t, where E_t is the smallest
//     integer (never decreasing) that keeps the tile's row maximum within
//     log2(448/256) of it, and the P V MFMA takes the per-lane block scale
//     2^E_t of the f8f6f4 instruction, so O accumulates p * 2^8 * 2^E_t
//     relative to m0 exactly.  Two row sums follow it: lq over the e4m3
//     values the product used (O = acc / lq, so a row whose weight sits on
//     one key is not off by that key's rounding, up to 2^-4), and l, the
//     lanes' fp32 sums of p before rounding times 2^E_t (the LSE).  Both
//     carry the same 2^8, which cancels in O and is removed from the LSE.
//     Only if E passes 64 (scores rising more than 64 log2 units above
//     tile 0) are O and the sums renormalised, to keep fp32 headroom.
//
// The vector work of the softmax per 64-key tile and 32 query rows (32
// exponentials, 16 e4m3 packs, 32 scale FMAs, 32 sums and the 16-instruction
// tile maximum) takes more issue time than the tile's nine matrix
// instructions: one wave issues a v_exp_f32 only every ~16 cycles, against
// ~8.6 for the SIMD as a whole, and exponentials and FMAs share issue (the
// issue-rate probes, fa_probe_rates.hip).  So a wave does its tiles in
// order (scores, tile maximum and E, exponentials and packs, P V) and three
// waves per SIMD hide each other's latencies; a software pipeline inside one
// wave (scores of tile t+1 and P V of tile t-1 around the softmax of tile t)
// needs ~250 registers and so allows only two waves, and measured 6-7%
// slower.  With at most 168 registers per wave: no second score buffer, P
// formed and consumed in the same tile, operand fragments read one product
// ahead, and the row sums of the rounded P from one 16x16x128 MFMA.
#include "fa_common.h"
#include "fa_exp2_fma.h"

namespace fa {

namespace {

constexpr int D = 128;
constexpr int BT = 64;               // keys per tile
constexpr int NCH = D / 16;          // 16-byte chunks per row (8)
constexpr float P_SHIFT = 8.0f;      // P is stored as p * 2^8
// p * 2^8 <= 448 (largest finite e4m3) when the score is at most
// log2(448 / 256) = 0.807 log2 units above the reference.
constexpr float P_HEADROOM = 0.8f;
constexpr int E_RENORM = 64;         // renormalise O, l beyond this shift

typedef __attribute__((ext_vector_type(2))) int i32x2_t;

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
                                            uint32_t voffset,
                                            uint32_t soffset = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)(dst), 16, voffset,
      soffset, 0, 0);
}

// The kernel (three waves per SIMD, design above):
//   * Workgroup: 4 waves x 32 rows (BR = 128), three workgroups per CU
//     (32 KB of LDS each).  K and V tiles of 64 keys are copied into LDS by
//     DMA one tile ahead (double-buffered): at the start of tile t every
//     wave waits for its copies of tile t, meets the others at the barrier
//     (so stage (t+1) % 2, tile t-1's, is free) and starts those of t+1.
//   * Row sum of the rounded P from v_mfma_scale_f32_16x16x128_f8f6f4 with
//     B = the lane's 32 packed P bytes.  In that product lane l supplies
//     column l % 16 of B (and row l % 16 of A) with k in [16 j, 16 j + 16)
//     (registers 0-3) and [64 + 16 j, 64 + 16 j + 16) (registers 4-7),
//     j = l / 16 (measured with one-hot operands); lane l of P holds query
//     l % 32, key half l / 32.  A = ones in lanes 0 and 32 (row 0) and 17
//     and 49 (row 1) gives C[0][n] = lq(query n) and C[1][n] = lq(query
//     n + 16), both in lane n < 16.  The E8M0 scale of k block b of column n
//     is taken from lane n + 16 b, which mixes queries n and n + 16, so this
//     product runs with neutral scales: it sums the rounded P as formed
//     (relative to m0 + E) while E stays put, and whenever some row's E
//     moves the sums are folded into fp32 totals times 2^E first.
//   * FMAP (0, 4, 8 or 16) of the 16 exponential pairs a lane forms per
//     tile run on the FMA pipe (exp2_fma, fa_exp2_fma.h) instead of
//     v_exp_f32; 0 is the default path.
template <bool CAUSAL, int FMAP>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(3, 3)))
fwd_fp8_kernel(const FwdArgs a) {
  static_assert(FMAP == 0 || FMAP == 4 || FMAP == 8 || FMAP == 16,
                "FMA-pipe exponential pairs per tile");
  constexpr int NWAVE = 4;
  constexpr int BR = 32 * NWAVE;
  constexpr int NWIN = BT * NCH / (64 * NWAVE);
  static_assert(NWIN == 2, "two copy windows per tile and operand");
  constexpr uint32_t WIN_BYTES = 8 * NWAVE * D;
  __shared__ uint4 Ks0[BT * NCH];
  __shared__ uint4 Ks1[BT * NCH];
  __shared__ uint4 Vs0[BT * NCH];
  __shared__ uint4 Vs1[BT * NCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const float cs = a.scale * dq * dk * 1.4426950408889634f;
  const bool neg = cs < 0.f;
  const float c = fmaxf(fabsf(cs), 1e-30f);

  const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                      (static_cast<int64_t>(b) * a.H + hq) * N * D;
  const uint8_t* kp = static_cast<const uint8_t*>(a.k) +
                      (static_cast<int64_t>(b) * a.Hkv + hk) * N * D;
  const uint8_t* vp = static_cast<const uint8_t*>(a.v) +
                      (static_cast<int64_t>(b) * a.Hkv + hk) * N * D;

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

  uint32_t koff, voff;
  {
    const int slot = 64 * wave + lane;
    const int r = slot / NCH, p = slot % NCH;
    koff = static_cast<uint32_t>(r * D + 16 * kswz(r, p));
    voff = static_cast<uint32_t>(r * D + 16 * vswz(r, p));
  }

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kv_end + BT - 1) / BT;

  auto rsrc_at = [&](const uint8_t* base, int kv0) {
    const int rows = max(kv_end - kv0, 0);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(base + static_cast<int64_t>(kv0) * D), 0,
        rows * D, 0x00020000);
  };
  auto copy_tile = [&](int t, const uint4* ks, const uint4* vs) {
    const auto rk = rsrc_at(kp, t * BT);
    const auto rv = rsrc_at(vp, t * BT);
#pragma unroll
    for (int w = 0; w < NWIN; ++w) {
      copy_to_lds(rk, ks + 64 * (wave + NWAVE * w), koff, w * WIN_BYTES);
      copy_to_lds(rv, vs + 64 * (wave + NWAVE * w), voff, w * WIN_BYTES);
    }
  };

  auto kfrag = [&](const uint4* ks, int kb, int s) {
    const int r = 32 * kb + sigma(li);
    const uint4* row = ks + r * NCH;
    const uint4 k0 = row[kswz(r, 4 * h + 2 * s)];
    const uint4 k1 = row[kswz(r, 4 * h + 2 * s + 1)];
    return i32x8_t{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w,
                   (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
  };
  const int tr_g = lane >> 4;
  const int tr_R = (lane >> 1) & 7;
  const int tr_j = lane & 1;
  const int tr_c = 2 * (tr_g & 1) + tr_j;
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
  // Row sums of the rounded P since E last moved (lane n < 16: queries n,
  // n + 16), and their totals times 2^E.
  float lraw0 = 0.f, lraw1 = 0.f;
  float lq0 = 0.f, lq1 = 0.f;
  float m0 = 0.f;
  int e_cur = 0;
  float l_run = 0.f;

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
  auto over = [&](float x) { return fmaf(x, c, -m0) - P_HEADROOM; };
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

  // Scores of tile t from stage ks, masked where needed.
  // Operand fragments are read one product ahead (the three waves of a
  // SIMD cover the rest of the LDS latency), which bounds the registers
  // they take to two fragments.
  auto scores = [&](int t, const uint4* ks, f32x16_t (&s)[2]) {
    s[0] = f32x16_t{};
    s[1] = f32x16_t{};
    i32x8_t kf = kfrag(ks, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const i32x8_t kcur = kf;
      if (i + 1 < 4) kf = kfrag(ks, (i + 1) & 1, (i + 1) >> 1);
      s[i & 1] = mfma_f8(kcur, qf[i >> 1], s[i & 1]);
      asm volatile("" ::: "memory");
    }
    if (masked_at(t)) apply_mask(s, t * BT);
  };
  // Lane-dependent A operand of the row-sum product (see above).
  const int m16 = lane & 15;
  const int one = ((m16 == 0 && (lane & 16) == 0) ||
                   (m16 == 1 && (lane & 16) != 0))
                      ? 0x38383838
                      : 0;
  // P of tile t from its scores (E already settled), its row sums and
  // O += P V from stage vs.
  auto accumulate = [&](const f32x16_t (&s)[2], const uint4* vs) {
    const float moff = P_SHIFT - (m0 + static_cast<float>(e_cur));
    int pw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "=v"(pw[i]));
    float ls0, ls1;
    // The softmax's vector work is what bounds a tile (see above): while a
    // wave is in it, its instructions go before the other waves' (whose
    // matrix instructions need few issue cycles); measured 1.0-1.4% faster
    // than equal priorities, and 1% slower with the priority on the matrix
    // instructions instead.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int kb = q >> 3, r = 2 * (q & 7);
      const float x0 = fmaf(s[kb][r], c, moff);
      const float x1 = fmaf(s[kb][r + 1], c, moff);
      // Pairs q = 0, 16 / FMAP, 2 * 16 / FMAP, ... on the FMA pipe.
      const bool on_fma = FMAP > 0 && q % (FMAP > 0 ? 16 / FMAP : 1) == 0;
      const float e0 = on_fma ? exp2_fma(x0) : __builtin_amdgcn_exp2f(x0);
      const float e1 = on_fma ? exp2_fma(x1) : __builtin_amdgcn_exp2f(x1);
      pw[q >> 1] = pack_fp8x2(e0, e1, pw[q >> 1], q & 1);
      float& ls = (q & 1) ? ls1 : ls0;
      if (q < 2)
        ls = e0 + e1;
      else
        ls += e0 + e1;
      // Each pair is packed and summed before the next is formed (keeps
      // the live registers to one pair).
      asm volatile("" : "+v"(pw[q >> 1]), "+v"(ls));
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_setprio(0);
    const i32x8_t pp = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
    const int eb = 127 + e_cur;
    const i32x8_t ones = {one, one, one, one, one, one, one, one};
    // A fresh accumulator per tile (a large running C would be added to the
    // 64 products with the matrix core's own alignment); fp32 sums after.
    f32x4_t lt = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        ones, pp, f32x4_t{}, 0, 0, 0, 127, 0, 127);
    asm volatile("" : "+v"(lt));
    lraw0 += lt[0];
    lraw1 += lt[1];
    i32x8_t vf = vfrag(vs, 0);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const i32x8_t vcur = vf;
      if (db + 1 < 4) vf = vfrag(vs, db + 1);
      oacc[db] = mfma_f8_bscale(vcur, pp, oacc[db], eb);
      // Keeps the product here (the compiler would otherwise sink the four
      // of them into the next tile, keeping V and P live across it).
      asm volatile("" : "+v"(oacc[db])::"memory");
    }
    l_run += __builtin_ldexpf(ls0 + ls1, e_cur);
  };
  // E for a tile with these scores (the smallest integer, never falling,
  // that keeps the row maximum within P_HEADROOM of m0 + E); O, l and the
  // row sums move down by 2^E if E passes E_RENORM.
  // Folds the raw row sums into the totals at the current E (lane n < 16:
  // E of query n is its own, that of query n + 16 is lane n + 16's).
  auto fold_lq = [&]() {
    const int e_hi = __builtin_amdgcn_ds_bpermute(((lane & 15) + 16) << 2,
                                                  e_cur);
    lq0 += __builtin_ldexpf(lraw0, e_cur);
    lq1 += __builtin_ldexpf(lraw1, e_hi);
    lraw0 = 0.f;
    lraw1 = 0.f;
  };
  auto settle_e = [&](const f32x16_t (&s)[2]) {
    const float lmx = lane_max(s);
    if (__builtin_amdgcn_ballot_w64(over(lmx) > static_cast<float>(e_cur)) !=
        0) {
      fold_lq();
      e_cur = next_e(half_max(lmx), e_cur);
      if (__builtin_amdgcn_ballot_w64(e_cur > E_RENORM) != 0) {   // rare
        // Every row moves its base up by its own E; lq1 (lane n < 16)
        // belongs to query n + 16, whose E is lane n + 16's.
        const int sh = e_cur;
        const int sh_hi =
            __builtin_amdgcn_ds_bpermute(((lane & 15) + 16) << 2, sh);
        const float f = __builtin_ldexpf(1.0f, -sh);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= f;
        l_run *= f;
        lq0 *= f;
        lq1 = __builtin_ldexpf(lq1, -sh_hi);
        m0 += static_cast<float>(sh);
        e_cur = 0;
      }
    }
  };

  // Stages: tile t lives in Ks[t % 2] / Vs[t % 2].  Tiles 0 and 1 come
  // first, then pairs (t, t + 1) for even t; when the tile count is odd the
  // last pair's second tile (or tile 1 when there is one tile) is virtual:
  // its copies read zeros (the descriptors end at kv_end) and its scores are
  // masked, so its p are 0.  Every copy issued is waited for before its
  // tile is read, so none is in flight when the workgroup ends.
  copy_tile(0, Ks0, Vs0);
  wait_copies_and_sync();
  copy_tile(1, Ks1, Vs1);
  if constexpr (SERIAL_COPIES) wait_copies_and_sync();
  {
    // Tile 0 sets the base (every row sees key 0: finite for existing rows).
    f32x16_t s[2];
    scores(0, Ks0, s);
    const float mx = half_max(lane_max(s));
    m0 = (mx == -__builtin_inff()) ? 0.f : mx * c;
    accumulate(s, Vs0);
  }
  wait_copies_and_sync();
  if (2 < ntiles) copy_tile(2, Ks0, Vs0);
  if constexpr (SERIAL_COPIES) wait_copies_and_sync();
  {
    f32x16_t s[2];
    scores(1, Ks1, s);
    settle_e(s);
    accumulate(s, Vs1);
  }
  for (int t = 2; t < ntiles; t += 2) {
    wait_copies_and_sync();
    copy_tile(t + 1, Ks1, Vs1);
    if constexpr (SERIAL_COPIES) wait_copies_and_sync();
    {
      f32x16_t s[2];
      scores(t, Ks0, s);
      settle_e(s);
      accumulate(s, Vs0);
    }
    wait_copies_and_sync();
    if (t + 2 < ntiles) copy_tile(t + 2, Ks0, Vs0);
    if constexpr (SERIAL_COPIES) wait_copies_and_sync();
    {
      f32x16_t s[2];
      scores(t + 1, Ks1, s);
      settle_e(s);
      accumulate(s, Vs1);
    }
  }

  // Epilogue.  Lane n < 16 holds the totals of queries n and n + 16; lane
  // L needs that of query L % 32.
  fold_lq();
  const float l_tot = half_sum(l_run);
  const int src = (li & 15) << 2;
  const float lqa = __int_as_float(
      __builtin_amdgcn_ds_bpermute(src, __float_as_int(lq0)));
  const float lqb = __int_as_float(
      __builtin_amdgcn_ds_bpermute(src, __float_as_int(lq1)));
  const float lq_tot = (li < 16) ? lqa : lqb;
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

template <int FMAP>
static void launch_fmap(const FwdArgs& a, bool causal, int grid,
                        hipStream_t stream) {
  if (causal) {
    hipLaunchKernelGGL((fwd_fp8_kernel<true, FMAP>), dim3(grid), dim3(256), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((fwd_fp8_kernel<false, FMAP>), dim3(grid), dim3(256),
                       0, stream, a);
  }
}

// 2^x elementwise by exp2_fma (the FMA-pipe exponential), grid-stride.
__global__ void __launch_bounds__(256)
exp2_fma_kernel(const float* x, float* y,
                long long n) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x +
                     threadIdx.x;
       i < n; i += stride)
    y[i] = exp2_fma(x[i]);
}

}  // namespace

hipError_t launch_fwd_fp8(FwdArgs a, bool causal, int fma_pairs,
                          hipStream_t stream) {
  constexpr int BR = 128;
  a.nqb = static_cast<int>((static_cast<long long>(a.N) + BR - 1) / BR);
  const long long grid = static_cast<long long>(a.B) * a.H * a.nqb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  if (static_cast<long long>(a.N) * D > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  const int bh = a.B * a.H;
  a.xcd_chunk = causal ? (bh % 8 == 0) : (grid % 8 == 0);
  switch (fma_pairs) {
    case 0: launch_fmap<0>(a, causal, (int)grid, stream); break;
    case 4: launch_fmap<4>(a, causal, (int)grid, stream); break;
    case 8: launch_fmap<8>(a, causal, (int)grid, stream); break;
    case 16: launch_fmap<16>(a, causal, (int)grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_exp2_fma(const float* x, float* y, long long n,
                           hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  const int grid = static_cast<int>(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(exp2_fma_kernel, dim3(grid), dim3(256), 0, stream, x, y,
                     n);
  return hipGetLastError();
}

}  // namespace fa
