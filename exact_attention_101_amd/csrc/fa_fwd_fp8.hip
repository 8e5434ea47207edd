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
//     with neutral (2^0) block scales, fp32 accumulation.
//   * P is rounded to e4m3 after multiplying by 2^8 (p' = exp2(t - m + 8),
//     at most 256 < 448), which keeps small weights out of the e4m3
//     subnormal range; the running denominator carries the same factor, so
//     it cancels in O = acc / l and is removed from the LSE.
//   * Q stays in registers; K and V tiles of 64 keys are double-buffered in
//     LDS; V^T operands come from the transposing ds_read_b64_tr_b8.
#include "fa_common.h"

namespace fa {

namespace {

constexpr int D = 128;
constexpr int BR = 128;
constexpr int BC = 64;
constexpr int NTHR = 256;
constexpr int NCH = D / 16;          // 16-byte chunks per row (8)
constexpr int KROWS = NTHR / NCH;    // rows per load pass (32)
constexpr int KPASS = BC / KROWS;    // passes per tile (2)
constexpr float P_SHIFT = 8.0f;      // P is stored as p * 2^8

// K tile: lane i reads row sigma(i) (+32 kb); XOR term depends on i only.
__device__ __forceinline__ int kswz(int r, int c) {
  const int t = sigma(r & 31);
  return c ^ ((t & 7) ^ ((t >> 3) & 1));
}

// V tile: the 8 key rows of one transposing read differ in (r % 2,
// (r >> 1) % 4); XOR-ing the 32-byte segment with (r >> 1) % 4 spreads them
// over all banks.
__device__ __forceinline__ int vswz(int r, int c) {
  return c ^ (2 * ((r >> 1) & 3));
}

typedef __attribute__((ext_vector_type(2))) int i32x2_t;

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

template <bool CAUSAL>
__global__ void __launch_bounds__(NTHR, 2)
fwd_fp8_kernel(const FwdArgs a) {
  __shared__ uint4 Ks[2][BC * NCH];   // [key][d] bytes, swizzled
  __shared__ uint4 Vs[2][BC * NCH];   // [key][d] bytes, swizzled

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
  // product is handled by negating Q's codes (sign bit) on load.
  const float cs = a.scale * dq * dk * 1.4426950408889634f;
  const bool neg = cs < 0.f;
  const float c = fabsf(cs);

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

  // Staging registers: thread tid moves 16-byte chunk (tid % NCH) of rows
  // tid / NCH and tid / NCH + 32 of both K and V (KPASS == 2).
  static_assert(KPASS == 2, "staging below is written for two passes");
  uint4 k0s, k1s, v0s, v1s;
  const int kc = tid % NCH;
  const int kr = tid / NCH;

  auto load_tile = [&](int kv0) {
    // Rows past the end read row N-1 (always in bounds).  Their scores are
    // masked; their V values are zeroed so that P = 0 times V stays 0.
    const int r0 = kv0 + kr, r1 = r0 + KROWS;
    const int64_t o0 = static_cast<int64_t>(min(r0, N - 1)) * D + 16 * kc;
    const int64_t o1 = static_cast<int64_t>(min(r1, N - 1)) * D + 16 * kc;
    k0s = *reinterpret_cast<const uint4*>(kp + o0);
    k1s = *reinterpret_cast<const uint4*>(kp + o1);
    v0s = keep_if(*reinterpret_cast<const uint4*>(vp + o0), r0 < N);
    v1s = keep_if(*reinterpret_cast<const uint4*>(vp + o1), r1 < N);
  };
  auto store_tile = [&](int buf) {
    const int r0 = kr, r1 = kr + KROWS;
    Ks[buf][r0 * NCH + kswz(r0, kc)] = k0s;
    Ks[buf][r1 * NCH + kswz(r1, kc)] = k1s;
    Vs[buf][r0 * NCH + vswz(r0, kc)] = v0s;
    Vs[buf][r1 * NCH + vswz(r1, kc)] = v1s;
  };

  // Transposed V read, per lane: group g = lane / 16, lanes 2R + j of the
  // group read key row R (+ tile offsets) at bytes [32 db + 16 (g % 2) + 8 j,
  // +8).  Output lane i then holds 8 keys of d = 32 db + 16 (g % 2) + i.
  const int tr_g = lane >> 4;
  const int tr_R = (lane >> 1) & 7;
  const int tr_j = lane & 1;
  const int tr_c = 2 * (tr_g & 1) + tr_j;        // 8-byte unit in a 32-d block

  f32x16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16_t{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kv_end + BC - 1) / BC;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const int kv0 = t * BC;
    if (t + 1 < ntiles) load_tile(kv0 + BC);

    const bool skip = CAUSAL && (kv0 > qw0 + 31);
    if (!skip) {
      f32x16_t sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16_t{};
        const int r = 32 * kb + sigma(li);
        const uint4* row = &Ks[buf][r * NCH];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint4 k0 = row[kswz(r, 4 * h + 2 * s)];
          const uint4 k1 = row[kswz(r, 4 * h + 2 * s + 1)];
          const i32x8_t kk = {(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w,
                              (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
          sacc[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              kk, qf[s], sacc[kb], 0, 0, 0, 127, 0, 127);
        }
      }

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
      const float moff = P_SHIFT - m_use;

      // P^T in e4m3: byte e = 16 kb + r of this lane <-> key
      // 32 kb + 16 (r / 8) + 8 h + r % 8.
      float psum = 0.f;
      int pw[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float s = sacc[w >> 2][4 * (w & 3) + e];
          p[e] = (s == -__builtin_inff())
                     ? 0.f
                     : __builtin_amdgcn_exp2f(fmaf(s, c, moff));
          psum += p[e];
        }
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        pw[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], v, true);
      }
      const i32x8_t pb = {pw[0], pw[1], pw[2], pw[3],
                          pw[4], pw[5], pw[6], pw[7]};
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

      // O^T += V^T P^T: A operand byte e of lane half h <-> the same key as
      // the B operand: read t8 (bytes 8 t8 .. 8 t8 + 7) covers keys
      // 16 t8 + 8 h + R, R = 0..7.
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        int av[8];
#pragma unroll
        for (int t8 = 0; t8 < 4; ++t8) {
          const int r = 16 * t8 + 8 * h + tr_R;
          const int unit = 4 * db + tr_c;                  // 8-byte unit
          const uint8_t* p = reinterpret_cast<const uint8_t*>(
                                 &Vs[buf][r * NCH + vswz(r, unit >> 1)]) +
                             8 * (unit & 1);
          const i32x2_t x = lds_read_tr8(p);
          av[2 * t8] = x[0];
          av[2 * t8 + 1] = x[1];
        }
        const i32x8_t va = {av[0], av[1], av[2], av[3],
                            av[4], av[5], av[6], av[7]};
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            va, pb, oacc[db], 0, 0, 0, 127, 0, 127);
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  Accumulator row m <-> d = 32 db + m: lane half h holds runs
  // of 4 consecutive d at 32 db + 8 (r / 4) + 4 h.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = (l_tot > 0.f) ? dv / l_tot : 0.f;
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
                ? (m_run + __log2f(l_tot) - P_SHIFT) * 0.69314718055994531f
                : -__builtin_inff();
    }
  }
}

}  // namespace

hipError_t launch_fwd_fp8(FwdArgs a, bool causal, hipStream_t stream) {
  a.nqb = (a.N + BR - 1) / BR;
  const long long grid = static_cast<long long>(a.B) * a.H * a.nqb;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const int bh = a.B * a.H;
  a.xcd_chunk = causal ? (bh % 8 == 0) : (grid % 8 == 0);
  if (causal) {
    hipLaunchKernelGGL(fwd_fp8_kernel<true>, dim3((int)grid), dim3(NTHR), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL(fwd_fp8_kernel<false>, dim3((int)grid), dim3(NTHR), 0,
                       stream, a);
  }
  return hipGetLastError();
}

}  // namespace fa
