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
//     BC = 64 keys, double-buffered in LDS;
//   * scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16: the accumulator column is the query, so each
//     lane holds 32 scores of one query and the row max / row sum are
//     in-lane plus one exchange between the two lane halves;
//   * Q lives in registers as the B operand for the whole kernel; the
//     contraction over d is permuted so that lane half h holds the
//     contiguous d-range [h*D/2, (h+1)*D/2);
//   * K rows are loaded in sigma order (see fa_common.h), so the fp32 score
//     accumulator, converted to bf16, is directly the B operand of
//     O^T = V^T P^T; V stays in its [key][d] layout in LDS and the A operand
//     (V^T) is read with the transposing ds_read_b64_tr_b16;
//   * softmax in fp32 registers in the log2 domain: p = exp2(S*c - m) with
//     c = |scale| * log2(e) (one FMA + v_exp_f32 per score);
//   * LDS rows are XOR-swizzled at 16-byte granularity so the MFMA operand
//     reads are free of bank conflicts.
#include "fa_common.h"

namespace fa {

namespace {

constexpr int BR = 128;
constexpr int BC = 64;
constexpr int NTHR = 256;

// Physical 16-byte chunk of logical chunk c in K-tile row r (D/8 chunks per
// row).  Lane i of a wave reads row sigma(i) (+32 kb), so the XOR term seen
// by lane i is a function of i alone: (i & 15) for 16-chunk rows, and
// (i & 7) ^ ((i >> 3) & 1) for 8-chunk rows.  Either way 8 consecutive lanes
// (and, for 16-chunk rows, 16) hit distinct bank groups.
template <int NCH>
__device__ __forceinline__ int swz(int r, int c) {
  const int t = sigma(r & 31);
  if constexpr (NCH == 16) {
    return c ^ (t & 15);
  } else {
    return c ^ ((t & 7) ^ ((t >> 3) & 1));
  }
}

// V tile: row = key, 64-byte segments of the row are XOR-ed with the key's
// position inside its group of 4 (16-chunk rows) or with bit 1 of the key
// (8-chunk rows), so the 4 key rows read by one ds_read_b64_tr_b16 land in
// different banks.
template <int NCH>
__device__ __forceinline__ int vswz(int r, int c) {
  if constexpr (NCH == 16) {
    return c ^ (4 * (r & 3));
  } else {
    return c ^ (4 * ((r >> 1) & 1));
  }
}

typedef __attribute__((ext_vector_type(4))) short i16x4_t;

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

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NTHR, 2)
fwd_bf16_kernel(const FwdArgs a) {
  constexpr int NCH = D / 8;            // 16-byte chunks per K row
  constexpr int NDB = D / 32;           // 32-row blocks of d (PV MFMA M-dim)
  constexpr int NKS = D / 16;           // k-steps of the QK^T MFMA
  constexpr int KROWS = NTHR / NCH;     // K rows loaded per pass
  constexpr int KPASS = BC / KROWS;     // K loads per thread per tile

  __shared__ uint4 Ks[2][BC * NCH];     // [key][d], swizzled
  __shared__ uint4 Vs[2][BC * NCH];     // [key][d], swizzled

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  bf16x8_t qf[NKS];
  {
    const uint32_t flip = a.neg ? 0x80008000u : 0u;
    const bool ok = qrow < N;
    const uint16_t* src = qp + static_cast<int64_t>(ok ? qrow : N - 1) * D +
                          h * (D / 2);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const uint4 x = ldg16(src + 8 * s);
      uint4 u = ok ? x : make_uint4(0, 0, 0, 0);
      u.x ^= flip; u.y ^= flip; u.z ^= flip; u.w ^= flip;
      qf[s] = as_bf16x8(u);
    }
  }

  // ---- K/V tile staging (global -> registers -> LDS) ----
  // Thread tid moves 16-byte chunk (tid % NCH) of rows tid / NCH + i * KROWS
  // of both K and V: each group of NCH lanes reads one whole row.
  uint4 kst[KPASS];
  uint4 vst[KPASS];
  const int kc = tid % NCH;
  const int kr = tid / NCH;

  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < KPASS; ++i) {
      // Rows past the end read row N-1 (always in bounds) and are zeroed.
      const int r = kv0 + kr + i * KROWS;
      const int64_t off = static_cast<int64_t>(min(r, N - 1)) * D + 8 * kc;
      const uint4 kx = ldg16(kp + off);
      const uint4 vx = ldg16(vp + off);
      const uint4 z = make_uint4(0, 0, 0, 0);
      kst[i] = (r < N) ? kx : z;
      vst[i] = (r < N) ? vx : z;
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPASS; ++i) {
      const int r = kr + i * KROWS;
      Ks[buf][r * NCH + swz<NCH>(r, kc)] = kst[i];
      Vs[buf][r * NCH + vswz<NCH>(r, kc)] = vst[i];
    }
  };

  // Per-lane part of the transposed V read (see lds_read_tr16): lane
  // 16 g + 4 R + j reads key row R (+ the tile offsets) at d-chunk
  // 2 (g % 2) + (j & 1) of a 32-wide d block, half (j >> 1).  The output
  // lane then holds 4 keys of d = 32 db + sigma(lane % 32).
  const int tr_g = lane >> 4;
  const int tr_R = (lane >> 2) & 3;
  const int tr_j = lane & 3;
  const int tr_c = 2 * (tr_g & 1) + (tr_j & 1);       // + 4 db
  const int tr_half = 4 * (tr_j >> 1);                  // 16-bit elements

  // ---- running softmax state (per lane = per query; both halves agree) ----
  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16_t{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;                    // this lane's half of the row sum
  const float c = a.c;

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kv0 = t * BC;
    if (t + 1 < ntiles) load_tile(kv0 + BC);

    const bool skip = CAUSAL && (kv0 > qw0 + 31);   // whole tile masked
    if (!skip) {
      // S^T = K Q^T for two 32-key blocks.
      f32x16_t sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16_t{};
        const int r = 32 * kb + sigma(li);
        const uint4* row = &Ks[buf][r * NCH];
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const uint4 kk = row[swz<NCH>(r, h * (NCH / 2) + s)];
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(kk), qf[s], sacc[kb], 0, 0, 0);
        }
      }

      // Mask: lane half h holds keys 32kb + 16(r/8) + 8h + (r%8).
      const bool need_mask =
          (kv0 + BC > N) || (CAUSAL && kv0 + BC - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kb + 16 * (r >> 3) + 8 * h + (r & 7);
            const bool ok = key < N && (!CAUSAL || key <= qrow);
            if (!ok) sacc[kb][r] = -__builtin_inff();
          }
        }
      }

      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_tile = (mx == -__builtin_inff()) ? mx : mx * c;
      const float m_new = fmaxf(m_run, m_tile);
      const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;

      float psum = 0.f;
      bf16x8_t pb[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float s0 = sacc[kb][8 * u + 2 * e];
            const float s1 = sacc[kb][8 * u + 2 * e + 1];
            const float p0 = (s0 == -__builtin_inff())
                                 ? 0.f
                                 : __builtin_amdgcn_exp2f(fmaf(s0, c, -m_use));
            const float p1 = (s1 == -__builtin_inff())
                                 ? 0.f
                                 : __builtin_amdgcn_exp2f(fmaf(s1, c, -m_use));
            psum += p0 + p1;
            w[e] = pack_bf16x2(p0, p1);
          }
          pb[kb][u] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }
      }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

      // O^T += V^T P^T.  k-slot (h, e) of this 16-key step is key
      // 32 kb + 16 u + 8 h + e on both operands.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r0 = 32 * kb + 16 * u + 8 * h + tr_R;   // key row, t4 = 0
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const uint16_t* v0 = reinterpret_cast<const uint16_t*>(
                &Vs[buf][r0 * NCH + vswz<NCH>(r0, 4 * db + tr_c)]) + tr_half;
            const uint16_t* v1 = reinterpret_cast<const uint16_t*>(
                &Vs[buf][(r0 + 4) * NCH + vswz<NCH>(r0 + 4, 4 * db + tr_c)]) +
                tr_half;
            const i16x4_t lo = lds_read_tr16(v0);
            const i16x4_t hi = lds_read_tr16(v1);
            const bf16x8_t vv = __builtin_bit_cast(
                bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                vv, pb[kb][u], oacc[db], 0, 0, 0);
          }
        }
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l in bf16 (RNE), LSE in natural log ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (qrow < N) {
    uint16_t* op = static_cast<uint16_t*>(a.o) +
                   ((static_cast<int64_t>(b) * a.H + hq) * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
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
      float* lp = a.lse + (static_cast<int64_t>(b) * a.H + hq) * N + qrow;
      *lp = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * 0.69314718055994531f
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
