// Shared device helpers and launch descriptors for the gfx950 attention
// kernels.  Internal header (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Race-check build (-DFA_SERIAL_COPIES=1, libfa_serial.so): the forward
// kernels put a workgroup barrier before every batch of tile copies into
// LDS and wait for the copies and meet at a barrier again right after it,
// so no stage is read while a copy into it is in flight and none is
// overwritten while a wave may still read it.  Its outputs must equal the
// pipelined build's bit for bit; a difference is a synchronisation bug.
#ifndef FA_SERIAL_COPIES
#define FA_SERIAL_COPIES 0
#endif

namespace fa {

constexpr bool SERIAL_COPIES = FA_SERIAL_COPIES != 0;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

// Arguments of one forward launch.  Element strides are 64-bit.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* descale;   // fp8 only: {dQ, dK, dV} or nullptr
  int B, H, Hkv, N;
  int group;              // H / Hkv
  int nqb;                // number of query blocks
  float c;                // |scale| * log2(e): scores enter exp2 in log2 units
  float scale;            // signed scale (fp8 path folds descales into it)
  int neg;                // scale < 0: Q is negated on load so that c >= 0
  int xcd_chunk;          // 1: map workgroups to XCD-contiguous work ranges
  int persist;            // dense non-causal forward: workgroups loop over
                          // the B * H * nqb units (grid < units)
  // Variable-length / windowed launches only (unused otherwise): sequence b
  // owns query rows [cu_q[b], cu_q[b+1]) and key rows [cu_k[b], cu_k[b+1])
  // of tensors packed per head; window widths (-1 = unbounded).
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  int left, right;
  // Masked launches only: bit j % 32 of word j / 32 of a row says whether
  // key j is visible; mw words per row; batch and head strides in words
  // (0: one mask shared); total_q / total_k are Nq / Nk.
  const uint32_t* mask;
  long long mask_bs, mask_hs;
  int mw;
};

// Arguments of one backward pass (bf16, d = 128).  ws holds, per query row
// (b, h, i), the pair {LSE_i * log2(e), D_i = dO_i . O_i}, written by the
// preprocessing kernel and read by both gradient kernels.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* ws;              // [B, H, N, 2]
  int B, H, Hkv, N;
  int group;              // H / Hkv
  int nqb;                // query blocks (dQ kernel)
  int nkb;                // key blocks (dK / dV kernel)
  float c;                // scale * log2(e), signed
  float scale;            // signed
  int xcd_chunk;          // as in FwdArgs, for the dQ kernel's grid
};

// Arguments of one split-KV forward (bf16, d = 128, Nq queries against Nk
// keys).  The workspace holds each split's normalised partial output
// (fp32, ws_o[s][row][d]) and its log2-unit LSE (ws_lse[s][row]), rows
// ordered (b, h, query).
constexpr int SPLITKV_MAX_SPLITS = 256;
// Floats of the per-device scratch that fa_fwd_splitkv_noalloc uses in place
// of a caller workspace: num_splits * B * H * Nq * (d + 1) must fit (16 MiB).
constexpr long long SPLITKV_SCRATCH_FLOATS = 4LL << 20;
struct SplitArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* ws_o;
  float* ws_lse;
  int B, H, Hkv, Nq, Nk;
  int group;              // H / Hkv
  int splits;
  int nrb;                // 32-row blocks per KV head (Nq * group rows)
  long long items;        // B * Hkv * nrb * splits waves
  long long rows_total;   // B * H * Nq
  float c;                // scale * log2(e), signed
};

// Arguments of one variable-length / sliding-window forward (bf16, d =
// 128).  Rows of all sequences are packed per head: q, o [H][total_q][d],
// k, v [Hkv][total_k][d], lse [H][total_q]; cu_q / cu_k hold B + 1 row
// offsets (device memory).
struct VarlenArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* cu_q;
  const int* cu_k;
  int B, H, Hkv;
  int group;              // H / Hkv
  int total_q, total_k;
  int max_q;              // longest query sequence (grid size)
  int nqb;                // 128-row query blocks of the longest sequence
  int left, right;        // window widths, -1 = unbounded (causal: right 0)
  float c;                // scale * log2(e), signed
};

constexpr int MASK_MAX_NK = 262144;   // keys a mask may cover (masked forward)
// Variable-length windows with left + right below this many keys (both
// bounded) run on the 128-row kernel, wider ones on the pipelined kernel.
constexpr int VARLEN_NARROW = 512;
// Packed rows per head a variable-length batch may hold (queries or keys):
// row, offset and window sums then stay below 2^31.
constexpr int VARLEN_MAX_ROWS = 1 << 29;

// x if ok, else zero; selected per 32-bit component (a select of the whole
// vector can end up in private memory).
__device__ __forceinline__ uint4 keep_if(uint4 x, bool ok) {
  return make_uint4(ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u,
                    ok ? x.w : 0u);
}

// Within a 32-row MFMA block, swap bits 2 and 3 of the row index.  Loading
// the A operand of S^T = K Q^T with key rows in this order makes every lane
// of the 32x32 accumulator hold 8 consecutive keys per half (keys 8h..8h+7
// and 16+8h..16+8h+7 of the block for lane half h), which is exactly the
// k-ordering the B operand of the following P V product wants.  It is an
// involution.
__device__ __forceinline__ int sigma(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Work-unit mapping.  Workgroup ids are dispatched round-robin over the 8
// XCDs (id % 8), each with its own L2.  Give each XCD a contiguous range of
// work so the query blocks that share one (batch, KV head) run on the same
// XCD and reuse K/V from its L2.  Causal launches go heaviest query block
// first (longest-processing-time order) inside each XCD's range.
__device__ __forceinline__ void map_work(int L, int T, int BH, int nqb,
                                         bool causal, int xcd_chunk, int& bh,
                                         int& qb) {
  if (xcd_chunk) {
    const int per = T >> 3;
    const int x = L & 7;
    const int s = L >> 3;
    if (causal) {
      const int hpx = BH >> 3;           // heads per XCD (BH % 8 == 0)
      bh = x * hpx + s % hpx;
      qb = nqb - 1 - s / hpx;
    } else {
      const int W = x * per + s;
      bh = W / nqb;
      qb = W % nqb;
    }
  } else {
    if (causal) {
      bh = L % BH;
      qb = nqb - 1 - L / BH;
    } else {
      bh = L / nqb;
      qb = L % nqb;
    }
  }
}

}  // namespace fa
