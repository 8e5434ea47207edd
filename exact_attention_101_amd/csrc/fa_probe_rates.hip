// Issue-rate probes for gfx950 (MI355X): how many cycles of a SIMD one
// wave64 instruction of each kind the softmax and the matrix products use
// occupies, alone and mixed, at 1 to 4 waves per SIMD.  Built into its own
// library (libfa_probe.so), not into libfa.so: it is measurement support for
// the attention kernels' roofline, not part of the attention path.
//
// The question it answers is the one the FlashAttention-4 article
// («Оптимизируйте производительность с FlashAttention-4», paragraph 3)
// raises for Blackwell: whether the exponential unit, rather than the matrix
// cores, bounds the forward, and whether computing some exponentials with
// ordinary FMA instructions would pay.  On this chip that depends on the
// cost of v_exp_f32 against v_fma_f32 on the same SIMD and on whether the
// two overlap, which the probes measure.
//
// Each wave runs `iters` rounds of one block of independent instructions
// (16 VALU instructions over 16 independent chains, or 4 MFMAs into 4
// accumulators) written as inline assembly or builtins the compiler cannot
// fold, between two reads of the shader clock (s_memtime) and of the
// 100 MHz reference clock (s_memrealtime).  The waves of one workgroup run
// one of two bodies each (the first 4 * na waves body A, the rest body B;
// wave w sits on SIMD w % 4), one workgroup per CU (it reserves 96 KiB of
// LDS).  Nothing is written but the per-wave timings.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_probe.h"
#include "fa_exp2_fma.h"

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) short short4_t;

enum Body {
  B_IDLE = 0,     // no work
  B_FMA = 1,      // 16 x v_fma_f32
  B_EXP = 2,      // 16 x v_exp_f32
  B_EXP_FMA = 3,  // 8 x v_exp_f32 interleaved with 8 x v_fma_f32
  B_CVT8 = 4,     // 16 x v_cvt_pk_fp8_f32
  B_MAX3 = 5,     // 16 x v_maximum3_f32
  B_ADD = 6,      // 16 x v_add_f32
  B_MFMA8 = 7,    // 4 x v_mfma_scale_f32_32x32x64_f8f6f4
  B_MFMA16 = 8,   // 4 x v_mfma_f32_32x32x16_bf16
  B_MFMA8_EXP = 9,    // 1 f8 MFMA + 8 exp + 8 fma (one softmax slot)
  B_MFMA16_EXP = 10,  // 1 bf16 MFMA + 4 exp + 4 fma
  B_EXP_CHAIN = 11,   // 4 x (v_fma_f32 -> v_exp_f32 -> v_add_f32), + 4 adds
  // MFMAs on operands from the caller's data (random values): 2 A and 2 B
  // fragments paired so that an operand changes from one MFMA to the next
  // as in a real product (switching activity sets the power drawn), few
  // enough to stay in registers beside the 4 accumulators.
  B_MFMA16_DATA = 12,  // 4 x v_mfma_f32_32x32x16_bf16
  B_MFMA8_DATA = 13,   // 4 x v_mfma_scale_f32_32x32x64_f8f6f4
  // Candidate softmax instructions of the bf16 kernel, alone and beside the
  // same wave's bf16 MFMAs (4 of them per MFMA).
  B_DOT2 = 14,         // 16 x v_dot2c_f32_bf16
  B_MOV64 = 15,        // 16 x v_mov_b64
  B_CVT16 = 16,        // 16 x v_cvt_pk_bf16_f32
  B_MFMA16_ADD = 17,   // 4 x (bf16 MFMA + 4 v_add_f32)
  B_MFMA16_DOT2 = 18,  // 4 x (bf16 MFMA + 4 v_dot2c_f32_bf16)
  B_MFMA16_MOV64 = 19, // 4 x (bf16 MFMA + 4 v_mov_b64)
  B_CVT8S = 20,        // 16 x v_cvt_scalef32_pk_fp8_f32
  // The bf16 forward's issue slot, 4 per round: scores MFMA (vector
  // accumulator), 2 x (v_fma_f32 -> v_exp_f32), P V MFMA (accumulation
  // registers), then v_cvt_pk_bf16_f32 and 2 v_add_f32 of the two
  // exponentials.
  B_SLOT16 = 21,
  // LDS reads of the bf16 forward, one wave's share of a 32-key step:
  // 8 x ds_read_b128 at the K fragment addresses, 16 x ds_read_b64_tr_b16
  // at the V fragment addresses, 16 x ds_read_b64_tr_b16 at 64 consecutive
  // 8-byte units (no two lanes of a 16-lane group in one bank group).
  B_LDS_K = 22,
  B_LDS_V = 23,
  B_LDS_TRSEQ = 24,
  // The FMA-pipe exponential of the fp8 forward's option (fa_exp2_fma.h):
  // 16 per round, eight vector instructions each.
  B_EXP2_FMA = 25,
  // The same issue slot with the vector work pipelined across slots: the
  // FMAs of pair i + 1 and the exponentials of pair i follow the first
  // MFMA, the pack and sums of pair i - 1 the second, so no vector
  // instruction waits for a result of its own slot.
  B_SLOT16P = 26,
  // LDS-DMA tile copies (buffer_load_dwordx4 ... lds, 1 KB per wave each)
  // from the caller's 16 KB buffer (L2-resident) into a 1 KB slice of the
  // workgroup's LDS reserve, at most 8 left in flight after each round:
  // 16 copies alone, 4 x (bf16 MFMA + copy), and the bf16 slot (body 21)
  // with a copy after its first MFMA, as the forward's copy steps issue
  // them.
  B_COPY = 27,
  B_MFMA16_COPY = 28,
  B_SLOT16_COPY = 29,
};

struct Regs {
  float x[16];
  float y, z;
  int w[8];
  double dd[8], dsrc;       // 64-bit move targets and source (B_*MOV64)
  f32x16_t acc[4];
  i32x8_t da[2], db[2];     // data operands (B_MFMA*_DATA)
  float lsum;               // B_SLOT16 lane sum
  float cs;                 // B_SLOT16 scale (uniform)
  float px0, px1, pe0, pe1; // B_SLOT16P values carried between slots
  const uint8_t* lds;       // B_LDS_*: the workgroup's LDS reserve
  __amdgpu_buffer_rsrc_t src;  // B_*COPY: the caller's 16 KB buffer
  float* dst;                  // B_*COPY: this wave's 1 KB of LDS
};

__device__ __forceinline__ void fma16(Regs& r, int first, int n) {
#pragma unroll
  for (int i = first; i < first + n; ++i)
    asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(r.x[i]) : "v"(r.y), "v"(r.z));
}

__device__ __forceinline__ void exp16(Regs& r, int first, int n) {
#pragma unroll
  for (int i = first; i < first + n; ++i)
    asm volatile("v_exp_f32 %0, %0" : "+v"(r.x[i]));
}

__device__ __forceinline__ void dot2(Regs& r, int i) {
  asm volatile("v_dot2c_f32_bf16 %0, %1, %2"
               : "+v"(r.x[i]) : "v"(r.w[i & 7]), "v"(r.w[(i + 3) & 7]));
}

__device__ __forceinline__ void mov64(Regs& r, int i) {
  asm volatile("v_mov_b64 %0, %1" : "=v"(r.dd[i & 7]) : "v"(r.dsrc));
}

template <int BODY>
__device__ __forceinline__ void round_of(Regs& r, const i32x8_t& a8,
                                         const bf16x8_t& a16) {
  if constexpr (BODY == B_FMA) {
    fma16(r, 0, 16);
  } else if constexpr (BODY == B_EXP) {
    exp16(r, 0, 16);
  } else if constexpr (BODY == B_EXP_FMA) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      asm volatile("v_exp_f32 %0, %0" : "+v"(r.x[i]));
      asm volatile("v_fma_f32 %0, %0, %1, %2"
                   : "+v"(r.x[8 + i]) : "v"(r.y), "v"(r.z));
    }
  } else if constexpr (BODY == B_CVT8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      asm volatile("v_cvt_pk_fp8_f32 %0, %1, %2"
                   : "+v"(r.w[i]) : "v"(r.x[2 * i]), "v"(r.x[2 * i + 1]));
      asm volatile("v_cvt_pk_fp8_f32 %0, %1, %2 op_sel:[0,0,1]"
                   : "+v"(r.w[i]) : "v"(r.x[2 * i + 1]), "v"(r.x[2 * i]));
    }
  } else if constexpr (BODY == B_MAX3) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      asm volatile("v_maximum3_f32 %0, %0, %1, %2"
                   : "+v"(r.x[i]) : "v"(r.y), "v"(r.z));
  } else if constexpr (BODY == B_ADD) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      asm volatile("v_add_f32 %0, %0, %1" : "+v"(r.x[i]) : "v"(r.y));
  } else if constexpr (BODY == B_MFMA8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          a8, a8, r.acc[j], 0, 0, 0, 127, 0, 127);
      asm volatile("" : "+v"(r.acc[j]));
    }
  } else if constexpr (BODY == B_MFMA16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a16, a16, r.acc[j],
                                                         0, 0, 0);
      asm volatile("" : "+v"(r.acc[j]));
    }
  } else if constexpr (BODY == B_MFMA8_EXP) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          a8, a8, r.acc[j], 0, 0, 0, 127, 0, 127);
      asm volatile("" : "+v"(r.acc[j]));
      if (j % 2 == 0) {
        exp16(r, 0, 8);
      } else {
        fma16(r, 8, 8);
      }
    }
  } else if constexpr (BODY == B_MFMA16_EXP) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a16, a16, r.acc[j],
                                                         0, 0, 0);
      asm volatile("" : "+v"(r.acc[j]));
      exp16(r, 4 * j, 2);
      fma16(r, 4 * j + 2, 2);
    }
  } else if constexpr (BODY == B_MFMA16_DATA) {
    // Fragment j: A from half j/2 of da[j%2], B from half j%2 of db[j/2].
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const i32x8_t ra = r.da[j & 1], rb = r.db[j >> 1];
      const bf16x8_t a = __builtin_bit_cast(
          bf16x8_t, (j >> 1) ? __builtin_shufflevector(ra, ra, 4, 5, 6, 7)
                             : __builtin_shufflevector(ra, ra, 0, 1, 2, 3));
      const bf16x8_t b = __builtin_bit_cast(
          bf16x8_t, (j & 1) ? __builtin_shufflevector(rb, rb, 4, 5, 6, 7)
                            : __builtin_shufflevector(rb, rb, 0, 1, 2, 3));
      r.acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, r.acc[j], 0, 0,
                                                         0);
      asm volatile("" : "+v"(r.acc[j]));
    }
  } else if constexpr (BODY == B_MFMA8_DATA) {
    // Operand pairs (da[0], db[0]), (da[1], db[0]), (da[0], db[1]),
    // (da[1], db[1]): one operand changes from each MFMA to the next.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          r.da[j & 1], r.db[j >> 1], r.acc[j], 0, 0, 0, 127, 0, 127);
      asm volatile("" : "+v"(r.acc[j]));
    }
  } else if constexpr (BODY == B_DOT2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) dot2(r, i);
  } else if constexpr (BODY == B_MOV64) {
#pragma unroll
    for (int i = 0; i < 16; ++i) mov64(r, i);
  } else if constexpr (BODY == B_CVT8S) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      typedef __attribute__((ext_vector_type(2))) short s2_t;
      s2_t o = __builtin_bit_cast(s2_t, r.w[i & 7]);
      if (i & 8)
        o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, r.x[i],
                                                    r.x[(i + 1) & 15], r.y,
                                                    true);
      else
        o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, r.x[i],
                                                    r.x[(i + 1) & 15], r.y,
                                                    false);
      r.w[i & 7] = __builtin_bit_cast(int, o);
      asm volatile("" : "+v"(r.w[i & 7]));
    }
  } else if constexpr (BODY == B_CVT16) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2"
                   : "=v"(r.w[i & 7]) : "v"(r.x[i]), "v"(r.x[(i + 1) & 15]));
  } else if constexpr (BODY == B_MFMA16_ADD || BODY == B_MFMA16_DOT2 ||
                       BODY == B_MFMA16_MOV64) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a16, a16, r.acc[j],
                                                         0, 0, 0);
      asm volatile("" : "+v"(r.acc[j]));
#pragma unroll
      for (int i = 4 * j; i < 4 * j + 4; ++i) {
        if constexpr (BODY == B_MFMA16_ADD)
          asm volatile("v_add_f32 %0, %0, %1" : "+v"(r.x[i]) : "v"(r.y));
        else if constexpr (BODY == B_MFMA16_DOT2)
          dot2(r, i);
        else
          mov64(r, i);
      }
    }
  } else if constexpr (BODY == B_SLOT16) {
    // Phases fenced as in the forward kernel; the scale is an opaque
    // scalar, so the FMAs read fixed inputs without being hoisted.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float cs = r.cs;
      asm volatile("" : "+s"(cs));
      __builtin_amdgcn_sched_barrier(0);
      r.acc[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          a16, a16, r.acc[j & 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      const float e0 = __builtin_amdgcn_exp2f(fmaf(r.x[2 * j], cs, -r.z));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(r.x[2 * j + 1], cs, -r.z));
      asm volatile("" : "+v"(r.acc[j & 1]));
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                   : "+a"(r.acc[2 + (j & 1)])
                   : "v"(a16), "v"(a16));
      __builtin_amdgcn_sched_barrier(0);
      bf16x2_t pk = {static_cast<__bf16>(e0), static_cast<__bf16>(e1)};
      r.w[j] = __builtin_bit_cast(int, pk);
      r.lsum += e0 + e1;
      asm volatile("" : "+v"(r.w[j]), "+v"(r.lsum));
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (BODY == B_SLOT16_COPY) {
    // Phases fenced as in the forward kernel; the scale is an opaque
    // scalar, so the FMAs read fixed inputs without being hoisted.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float cs = r.cs;
      asm volatile("" : "+s"(cs));
      __builtin_amdgcn_sched_barrier(0);
      r.acc[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          a16, a16, r.acc[j & 1], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r.src, (__attribute__((address_space(3))) void*)(r.dst), 16,
          16 * (threadIdx.x & 63), 1024 * j, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      const float e0 = __builtin_amdgcn_exp2f(fmaf(r.x[2 * j], cs, -r.z));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(r.x[2 * j + 1], cs, -r.z));
      asm volatile("" : "+v"(r.acc[j & 1]));
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                   : "+a"(r.acc[2 + (j & 1)])
                   : "v"(a16), "v"(a16));
      __builtin_amdgcn_sched_barrier(0);
      bf16x2_t pk = {static_cast<__bf16>(e0), static_cast<__bf16>(e1)};
      r.w[j] = __builtin_bit_cast(int, pk);
      r.lsum += e0 + e1;
      asm volatile("" : "+v"(r.w[j]), "+v"(r.lsum));
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8)
  } else if constexpr (BODY == B_COPY) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r.src, (__attribute__((address_space(3))) void*)(r.dst), 16,
          16 * (threadIdx.x & 63), 1024 * j, 0, 0);
    __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8)
  } else if constexpr (BODY == B_MFMA16_COPY) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a16, a16, r.acc[j],
                                                         0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r.src, (__attribute__((address_space(3))) void*)(r.dst), 16,
          16 * (threadIdx.x & 63), 1024 * j, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt(8)
  } else if constexpr (BODY == B_SLOT16P) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float cs = r.cs;
      asm volatile("" : "+s"(cs));
      __builtin_amdgcn_sched_barrier(0);
      r.acc[j & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          a16, a16, r.acc[j & 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      const float nx0 = fmaf(r.x[(2 * j + 2) & 15], cs, -r.z);
      const float nx1 = fmaf(r.x[(2 * j + 3) & 15], cs, -r.z);
      const float e0 = __builtin_amdgcn_exp2f(r.px0);
      const float e1 = __builtin_amdgcn_exp2f(r.px1);
      asm volatile("" : "+v"(r.acc[j & 1]));
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                   : "+a"(r.acc[2 + (j & 1)])
                   : "v"(a16), "v"(a16));
      __builtin_amdgcn_sched_barrier(0);
      bf16x2_t pk = {static_cast<__bf16>(r.pe0), static_cast<__bf16>(r.pe1)};
      r.w[j] = __builtin_bit_cast(int, pk);
      r.lsum += r.pe0 + r.pe1;
      asm volatile("" : "+v"(r.w[j]), "+v"(r.lsum));
      __builtin_amdgcn_sched_barrier(0);
      r.px0 = nx0;
      r.px1 = nx1;
      r.pe0 = e0;
      r.pe1 = e1;
    }
  } else if constexpr (BODY == B_LDS_K || BODY == B_LDS_V ||
                       BODY == B_LDS_TRSEQ) {
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
    typedef __attribute__((address_space(3))) const u32x4_t lds_u4;
    typedef __attribute__((address_space(3))) short4_t lds_s4;
    const int lane = threadIdx.x & 63;
    const int li = lane & 31, hh = lane >> 5;
    if constexpr (BODY == B_LDS_K) {
      // Rows of 17 16-byte slots; lane row sigma(li), chunk 8 hh + s.
      const int m = li;
      const int sg = (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
      const int base = (sg * 17 + hh * 8) * 16;
      u32x4_t k[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        k[i] = *(lds_u4*)(r.lds + base + 16 * i);
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(k[i]));
    } else {
      int base;
      if constexpr (BODY == B_LDS_V) {
        // Unpadded 256-byte rows, 64-byte segment XOR (row % 4).
        const int R = (lane >> 2) & 3, j = lane & 3;
        const int row = 8 * hh + R;
        const int ch = 4 * (row & 3) + 2 * ((lane >> 4) & 1) + (j & 1);
        base = (row * 16 + ch) * 16 + 8 * (j >> 1);
      } else {
        base = 8 * lane;
      }
      short4_t v[16];
#pragma unroll
      for (int f = 0; f < 8; ++f) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int off = BODY == B_LDS_V
                              ? ((base ^ ((f % 4) << 6)) +
                                 (16 * (f / 4) + 4 * hf) * 256)
                              : base + 512 * (2 * f + hf);
          v[2 * f + hf] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s4*)(r.lds + off));
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(v[i]));
    }
  } else if constexpr (BODY == B_EXP2_FMA) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      r.x[i] = fa::exp2_fma(r.x[i]);
      asm volatile("" : "+v"(r.x[i]));
    }
  } else if constexpr (BODY == B_EXP_CHAIN) {
    // The softmax's dependent sequence: scale and shift, exponential, sum.
    // Written with builtins so that the compiler inserts the wait states a
    // use of a transcendental result needs.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float t = __builtin_amdgcn_exp2f(fmaf(r.x[i], r.y, r.z));
      r.x[8 + i] += t;
      asm volatile("" : "+v"(r.x[8 + i]));
      r.x[i] += 1.0f;
      asm volatile("" : "+v"(r.x[i]));
    }
  }
}

template <int BODY>
__device__ __forceinline__ void run(Regs& r, int iters, const i32x8_t& a8,
                                    const bf16x8_t& a16) {
  for (int it = 0; it < iters; ++it) round_of<BODY>(r, a8, a16);
}

template <int A, int B>
__global__ void __launch_bounds__(1024) probe_kernel(unsigned long long* out,
                                                     const i32x8_t* data,
                                                     int iters, int na,
                                                     float seed) {
  __shared__ float reserve[24576];      // 96 KiB: one workgroup per CU
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  Regs r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r.x[i] = seed * (i + 1) + 1e-3f * lane;
  r.y = 0.999f;
  r.z = seed;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.w[i] = 0x3F803F80 + i;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.dd[i] = seed * i;
  r.dsrc = seed;
  r.lsum = 0.f;
  r.cs = 0.999f;
  r.px0 = r.px1 = r.pe0 = r.pe1 = seed;
  r.lds = reinterpret_cast<const uint8_t*>(reserve);
  r.src = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<i32x8_t*>(data), 0, data ? 16384 : 0, 0x00020000);
  r.dst = reserve + 256 * __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
  for (int j = 0; j < 4; ++j) r.acc[j] = f32x16_t{};
  // Data operands: lane-dependent fragments of the caller's 512-entry
  // buffer (all zeros when no buffer is given).
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    r.da[j] = data ? data[(lane + 64 * j) & 511] : i32x8_t{};
    r.db[j] = data ? data[(lane + 64 * j + 256) & 511] : i32x8_t{};
  }
  const int s8 = 0x38383838 + (lane & 1);   // e4m3 codes near 1.0
  const i32x8_t a8 = {s8, s8, s8, s8, s8, s8, s8, s8};
  bf16x8_t a16;
#pragma unroll
  for (int i = 0; i < 8; ++i) a16[i] = static_cast<__bf16>(seed + 0.5f * i);

  __syncthreads();
  const uint64_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  if ((wave >> 2) < na)
    run<A>(r, iters, a8, a16);
  else
    run<B>(r, iters, a8, a16);
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();

  // Keep every result alive (never true for the seeds used).
  float sink = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sink += r.x[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) sink += static_cast<float>(r.w[i]);
#pragma unroll
  for (int i = 0; i < 8; ++i) sink += static_cast<float>(r.dd[i]);
#pragma unroll
  for (int j = 0; j < 4; ++j) sink += r.acc[j][lane & 15];
  sink += r.lsum + r.px0 + r.px1 + r.pe0 + r.pe1;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    sink += static_cast<float>(r.da[j][lane & 7] ^ r.db[j][lane & 7]);
  if (iters < 0) {
    reserve[tid] = sink;
    __syncthreads();
    out[0] = static_cast<unsigned long long>(reserve[(tid + 1) & 1023]);
  }
  if (lane == 0) {
    const size_t g = (static_cast<size_t>(blockIdx.x) * (blockDim.x >> 6) +
                      wave) * 3;
    out[g + 0] = t1 - t0;
    out[g + 1] = r1 - r0;
    out[g + 2] = hw;
  }
}

template <int A, int B>
hipError_t launch(unsigned long long* out, const i32x8_t* data, int iters,
                  int na, int waves, int grid, hipStream_t s) {
  hipLaunchKernelGGL((probe_kernel<A, B>), dim3(grid), dim3(64 * waves), 0, s,
                     out, data, iters, na, 1.0e-3f);
  return hipGetLastError();
}

typedef hipError_t (*launch_fn)(unsigned long long*, const i32x8_t*, int, int,
                                int, int, hipStream_t);

template <int A>
launch_fn pick_b(int b) {
  switch (b) {
    case B_IDLE: return launch<A, B_IDLE>;
    case B_FMA: return launch<A, B_FMA>;
    case B_EXP: return launch<A, B_EXP>;
    case B_EXP_FMA: return launch<A, B_EXP_FMA>;
    case B_CVT8: return launch<A, B_CVT8>;
    case B_MAX3: return launch<A, B_MAX3>;
    case B_ADD: return launch<A, B_ADD>;
    case B_MFMA8: return launch<A, B_MFMA8>;
    case B_MFMA16: return launch<A, B_MFMA16>;
    case B_MFMA8_EXP: return launch<A, B_MFMA8_EXP>;
    case B_MFMA16_EXP: return launch<A, B_MFMA16_EXP>;
    case B_EXP_CHAIN: return launch<A, B_EXP_CHAIN>;
    case B_DOT2: return launch<A, B_DOT2>;
    case B_MOV64: return launch<A, B_MOV64>;
    case B_CVT16: return launch<A, B_CVT16>;
    case B_CVT8S: return launch<A, B_CVT8S>;
    case B_EXP2_FMA: return launch<A, B_EXP2_FMA>;
    default: return nullptr;
  }
}

// Bodies that run alone (B idle): the data-operand MFMAs.
launch_fn pick_alone(int a) {
  switch (a) {
    case B_MFMA16_DATA: return launch<B_MFMA16_DATA, B_IDLE>;
    case B_MFMA8_DATA: return launch<B_MFMA8_DATA, B_IDLE>;
    case B_MFMA16_ADD: return launch<B_MFMA16_ADD, B_IDLE>;
    case B_MFMA16_DOT2: return launch<B_MFMA16_DOT2, B_IDLE>;
    case B_MFMA16_MOV64: return launch<B_MFMA16_MOV64, B_IDLE>;
    case B_SLOT16: return launch<B_SLOT16, B_IDLE>;
    case B_SLOT16P: return launch<B_SLOT16P, B_IDLE>;
    case B_COPY: return launch<B_COPY, B_IDLE>;
    case B_MFMA16_COPY: return launch<B_MFMA16_COPY, B_IDLE>;
    case B_SLOT16_COPY: return launch<B_SLOT16_COPY, B_IDLE>;
    case B_LDS_K: return launch<B_LDS_K, B_IDLE>;
    case B_LDS_V: return launch<B_LDS_V, B_IDLE>;
    case B_LDS_TRSEQ: return launch<B_LDS_TRSEQ, B_IDLE>;
    default: return nullptr;
  }
}

launch_fn pick(int a, int b) {
  switch (a) {
    case B_FMA: return pick_b<B_FMA>(b);
    case B_EXP: return pick_b<B_EXP>(b);
    case B_EXP_FMA: return pick_b<B_EXP_FMA>(b);
    case B_CVT8: return pick_b<B_CVT8>(b);
    case B_MAX3: return pick_b<B_MAX3>(b);
    case B_ADD: return pick_b<B_ADD>(b);
    case B_MFMA8: return pick_b<B_MFMA8>(b);
    case B_MFMA16: return pick_b<B_MFMA16>(b);
    case B_MFMA8_EXP: return pick_b<B_MFMA8_EXP>(b);
    case B_MFMA16_EXP: return pick_b<B_MFMA16_EXP>(b);
    case B_EXP_CHAIN: return pick_b<B_EXP_CHAIN>(b);
    case B_DOT2: return pick_b<B_DOT2>(b);
    case B_MOV64: return pick_b<B_MOV64>(b);
    case B_CVT16: return pick_b<B_CVT16>(b);
    case B_CVT8S: return pick_b<B_CVT8S>(b);
    case B_EXP2_FMA: return pick_b<B_EXP2_FMA>(b);
    case B_MFMA16_ADD: return b == B_IDLE ? pick_alone(a) : nullptr;
    case B_MFMA16_DOT2: return b == B_IDLE ? pick_alone(a) : nullptr;
    case B_MFMA16_MOV64: return b == B_IDLE ? pick_alone(a) : nullptr;
    case B_SLOT16:
    case B_SLOT16P:
    case B_COPY:
    case B_MFMA16_COPY:
    case B_SLOT16_COPY:
    case B_LDS_K:
    case B_LDS_V:
    case B_LDS_TRSEQ: return b == B_IDLE ? pick_alone(a) : nullptr;
    case B_MFMA16_DATA:
    case B_MFMA8_DATA: return b == B_IDLE ? pick_alone(a) : nullptr;
    default: return nullptr;
  }
}

// Streaming read of a device buffer: every thread issues eight 16-byte
// loads before it combines them (grid-stride), so a CU keeps hundreds of
// kilobytes in flight.  A thread writes its word only if the XOR of what it
// read equals a fixed pattern, which keeps the loads without a store per
// thread.
typedef __attribute__((ext_vector_type(4))) unsigned u32x4v_t;
__global__ void __launch_bounds__(256) read_kernel(const u32x4v_t* src,
                                                   long long n,
                                                   unsigned* sink) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  unsigned acc = 0;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4v_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n; i += stride) {
    const u32x4v_t v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Contract in include/fa_probe.h.
extern "C" __attribute__((visibility("default"))) int fa_probe_rates(
    int a, int b, int waves, int na, int iters, int grid,
    unsigned long long* out, const void* data, void* stream) {
  if (!out || waves < 4 || waves > 16 || waves % 4 != 0 || na < 0 ||
      na > waves / 4 || iters < 1 || grid < 1)
    return 1;
  if ((a == B_MFMA16_DATA || a == B_MFMA8_DATA || a == B_COPY ||
       a == B_MFMA16_COPY || a == B_SLOT16_COPY) &&
      (!data || (reinterpret_cast<uintptr_t>(data) & 31u)))
    return 1;
  const launch_fn f = pick(a, b);
  if (!f) return 1;
  return f(out, static_cast<const i32x8_t*>(data), iters, na, waves, grid,
           static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? 0
             : 4;
}

// Contract in include/fa_probe.h.
extern "C" __attribute__((visibility("default"))) int fa_probe_read(
    const void* src, unsigned long long bytes, int grid, unsigned* sink,
    void* stream) {
  if (!src || !sink || grid < 1 || bytes == 0 || bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15u))
    return 1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream),
                     static_cast<const u32x4v_t*>(src),
                     static_cast<long long>(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
