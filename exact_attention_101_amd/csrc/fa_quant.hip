// FP8 input preparation for gfx950: optional random-sign Hadamard rotation
// of each 128-wide row ("incoherent processing", FlashAttention-3 summary
// (GeekNews), section «Baixa precisão: redução do erro de quantização com
// processamento incoerente») followed by per-tensor OCP e4m3 quantisation.
//
// Three stream-ordered kernels, no host synchronisation:
//   1. clear the amax cell;
//   2. rotate (if asked) and reduce max |x'| into it (atomic max on the
//      float's bit pattern, which orders like the value for x >= 0);
//   3. rotate again and write codes of x' * (448 / amax), rounded to nearest
//      even after clamping to +-448 (the e4m3 conversion does not saturate
//      on its own), plus the descale amax / 448.
// The pass is bound by HBM bandwidth: it reads the fp32 tensor twice and
// writes one byte per element.
//
// Row layout in a wave: 16 lanes per row, lane p of the group holds elements
// [8 p, 8 p + 8) (two 16-byte loads).  The fast Walsh-Hadamard transform
// runs its three distance-1/2/4 butterfly stages in registers and the four
// distance-8..64 stages across lanes of the 16-lane group.
#include "fa_common.h"

namespace fa {

namespace {

constexpr int QTHR = 256;
constexpr int ROWS_PER_BLOCK = QTHR / 16;   // 16 rows per workgroup pass

__global__ void clear_amax_kernel(float* amax_descale) {
  if (threadIdx.x == 0) amax_descale[0] = 0.f;
}

// Signs for elements [8 p, 8 p + 8): bit i of the 128-bit mask set means
// s_i = -1.
__device__ __forceinline__ void apply_signs(float (&x)[8], int p, uint64_t lo,
                                            uint64_t hi) {
  const uint64_t m = (p < 8) ? lo : hi;
  const int sh = 8 * (p & 7);
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if ((m >> (sh + e)) & 1ULL) x[e] = -x[e];
}

// x' = x diag(s) H_128 / sqrt(128) for the 128 elements spread over the 16
// lanes of a group (8 per lane).  Sylvester ordering: element index
// i = 8 p + e; a butterfly of distance 2^k pairs i with i ^ 2^k, the lower
// index keeping the sum and the upper the difference.
__device__ __forceinline__ void fwht128(float (&x)[8], int p) {
#pragma unroll
  for (int dist = 1; dist < 8; dist <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & dist) == 0) {
        const float a = x[e], b = x[e + dist];
        x[e] = a + b;
        x[e + dist] = a - b;
      }
    }
  }
#pragma unroll
  for (int ld = 1; ld < 16; ld <<= 1) {       // lane distance 1..8 = 8..64
    const bool upper = (p & ld) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float other = __shfl_xor(x[e], ld, 16);
      x[e] = upper ? (other - x[e]) : (x[e] + other);
    }
  }
  const float inv_sqrt = 0.088388347648318440550f;   // 1/sqrt(128)
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= inv_sqrt;
}

__device__ __forceinline__ void load_row8(const float* x, long long row, int p,
                                          float (&v)[8]) {
  const float4* src = reinterpret_cast<const float4*>(x + row * 128 + 8 * p);
  const float4 a = src[0], b = src[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__global__ void __launch_bounds__(QTHR)
amax_kernel(const float* __restrict__ x, float* amax_descale, long long rows,
            uint64_t lo, uint64_t hi, int rotate) {
  const int p = threadIdx.x & 15;
  const long long step = static_cast<long long>(gridDim.x) * ROWS_PER_BLOCK;
  float m = 0.f;
  for (long long row = static_cast<long long>(blockIdx.x) * ROWS_PER_BLOCK +
                       (threadIdx.x >> 4);
       row < rows; row += step) {
    float v[8];
    load_row8(x, row, p, v);
    if (rotate) {
      apply_signs(v, p, lo, hi);
      fwht128(v, p);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  }
  // The rows loop is uniform across each 16-lane group (rows are assigned
  // per group), so every lane of the wave reaches this reduction.
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wmax[QTHR / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float bm = wmax[0];
    for (int i = 1; i < QTHR / 64; ++i) bm = fmaxf(bm, wmax[i]);
    atomicMax(reinterpret_cast<unsigned int*>(amax_descale),
              __float_as_uint(bm));
  }
}

__global__ void __launch_bounds__(QTHR)
quant_kernel(const float* __restrict__ x, uint8_t* __restrict__ x8,
             float* amax_descale, long long rows, uint64_t lo, uint64_t hi,
             int rotate) {
  const float amax = amax_descale[0];
  const float inv = (amax > 0.f) ? 448.0f / amax : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0)
    amax_descale[1] = (amax > 0.f) ? amax / 448.0f : 1.0f;
  const int p = threadIdx.x & 15;
  const long long step = static_cast<long long>(gridDim.x) * ROWS_PER_BLOCK;
  for (long long row = static_cast<long long>(blockIdx.x) * ROWS_PER_BLOCK +
                       (threadIdx.x >> 4);
       row < rows; row += step) {
    float v[8];
    load_row8(x, row, p, v);
    if (rotate) {
      apply_signs(v, p, lo, hi);
      fwht128(v, p);
    }
    int w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y[e] = fminf(fmaxf(v[4 * k + e] * inv, -448.0f), 448.0f);
      const int t = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      w[k] = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], t, true);
    }
    *reinterpret_cast<uint2*>(x8 + row * 128 + 8 * p) =
        make_uint2(static_cast<unsigned>(w[0]), static_cast<unsigned>(w[1]));
  }
}

}  // namespace

hipError_t launch_fp8_quantize(const float* x, uint8_t* x8,
                               float* amax_descale, long long rows,
                               uint64_t sign_lo, uint64_t sign_hi, bool rotate,
                               hipStream_t stream) {
  long long blocks = (rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  if (blocks > 256 * 16) blocks = 256 * 16;   // grid-stride beyond 16 WG/CU
  hipLaunchKernelGGL(clear_amax_kernel, dim3(1), dim3(64), 0, stream,
                     amax_descale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(amax_kernel, dim3((int)blocks), dim3(QTHR), 0, stream, x,
                     amax_descale, rows, sign_lo, sign_hi, rotate ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quant_kernel, dim3((int)blocks), dim3(QTHR), 0, stream, x,
                     x8, amax_descale, rows, sign_lo, sign_hi,
                     rotate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace fa
