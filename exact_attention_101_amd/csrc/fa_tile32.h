// 32-row tiles of 128-wide bf16 rows streamed through LDS by four waves:
// copy plans, MFMA operand reads and O-shaped stores shared by the kernels
// that use one lane per row (the backward's gradient kernels and the
// masked / variable-length forward).  Internal header.
//
// LDS layouts of a 32-row tile (rows are keys or queries, 16-byte chunks):
//   row layout: row r = 8 g + i, chunk c stored at chunk 136 g + 8 c + i
//     (chunk-major within each 8-row group, groups 136 chunks apart): the
//     16 lanes that read chunk c of rows 0..15 (or 16..31) for a row
//     fragment hit 16 different 16-byte bank slots, and a k-step moves the
//     address by a constant;
//   transposed-read layout: row r, chunk c stored at chunk
//     r * 16 + ((c / 4) ^ (r % 4)) * 4 + c % 4, for ds_read_b64_tr_b16.
// Tiles arrive by buffer_load_dwordx4 ... lds, eight 64-lane copies per
// tile, two per wave, each reading whole 128-byte lines.  A wave's copies
// share one per-lane offset per layout; what differs between them goes into
// the buffer descriptor's base.  Rows past the descriptor's end read zeros.
#pragma once

#include "fa_common.h"

namespace fa {
namespace {

constexpr int D = 128;
constexpr int NCH = D / 8;                  // 16-byte chunks per row
constexpr int T = 32;                       // rows per tile (one step)
constexpr int NW = 4;                       // waves per workgroup
constexpr int NTHR = 64 * NW;
constexpr int BLK = T * NW;                 // rows per workgroup (128)
constexpr int RG = 136;                     // row layout: group stride
constexpr int ROW_ALLOC = 3 * RG + 8 * NCH; // 536 chunks, row layout
constexpr int TR_SLOTS = T * NCH;           // 512 chunks, transposed layout
constexpr int HALF_ROWS = 16;               // rows per descriptor
constexpr float LOG2E = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(4))) short i16x4_t;

__device__ __forceinline__ i16x4_t lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8_t, u);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t& a, const bf16x8_t& b,
                                         const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One 64-lane copy of 16 (copy16) or 4 (copy4) bytes per lane from `rsrc`
// + voffset into LDS at `dst` + that many bytes * lane.  Offsets past the
// descriptor's size read 0.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t rsrc,
                                       const void* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)(dst), 16, voffset, 0, 0,
      0);
}
__device__ __forceinline__ void copy4(__amdgpu_buffer_rsrc_t rsrc,
                                      const void* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)(dst), 4, voffset, 0, 0,
      0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base,
                                                            int64_t row0,
                                                            int rows,
                                                            int row_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(base) + row0 * row_bytes), 0,
      max(rows, 0) * row_bytes, 0x00020000);
}

// Per-lane global byte offsets of the two 64-lane copies one wave issues
// for each layout of a 32-row tile of 256-byte rows:
//   row layout, wave w, copy k: 8-row group w, chunks 8 k .. 8 k + 7; lane
//     L reads row 8 w + L % 8, chunk 8 k + L / 8 and writes LDS chunk
//     136 w + 64 k + L.  The descriptor starts at row 16 (w / 2) and, for
//     k = 1, 128 bytes further;
//   transposed layout, wave w, copy i: lane L reads row 4 w + 16 i + L / 16,
//     chunk c(L) with c's 4-chunk group swizzled by the row (row % 4 =
//     L / 16), and writes LDS chunk 256 i + 64 w + L.  The descriptor starts
//     at row 16 i.
struct TileCopy {
  uint32_t row_v;
  uint32_t tr_v;

  __device__ void init(int wave, int lane) {
    row_v = static_cast<uint32_t>((8 * (wave & 1) + (lane & 7)) * D * 2 +
                                  (lane >> 3) * 16);
    const int q = lane >> 4, p = lane & 15;
    const int c = (((p >> 2) ^ q) << 2) | (p & 3);
    tr_v = static_cast<uint32_t>((4 * wave + q) * D * 2 + c * 16);
  }

  // Copies of rows r0 .. r0 + 31 of `base` (rows_left rows exist from r0).
  __device__ void rows(const void* base, int r0, int rows_left,
                       const uint4* dst, int wave) const {
    const int h16 = HALF_ROWS * (wave >> 1);
    const int bytes = max(rows_left - h16, 0) * D * 2;
    const char* b = static_cast<const char*>(base) +
                    static_cast<int64_t>(r0 + h16) * D * 2;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      // readfirstlane keeps the (uniform) size scalar: a saturating
      // subtract would otherwise go to a vector register and force a
      // per-lane loop around the copy.
      const int rec = __builtin_amdgcn_readfirstlane(
          bytes > 128 * k ? bytes - 128 * k : 0);
      copy16(__builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(b + 128 * k),
                                               0, rec, 0x00020000),
             dst + RG * wave + 64 * k, row_v);
    }
  }
  __device__ void tr(const void* base, int r0, int rows_left,
                     const uint4* dst, int wave) const {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      copy16(rows_rsrc(base, r0 + HALF_ROWS * i, rows_left - HALF_ROWS * i,
                       D * 2),
             dst + 256 * i + 64 * wave, tr_v);
  }
};

// Byte offset, inside a transposed-read tile, of lane's first 8-byte read
// for d block 0 (see the forward kernel's V reads): lane 16 g + 4 R + j
// reads row 8 h + R at d = 16 (g % 2) + 8 (j % 2) + 4 (j / 2), and the
// output lane then holds 4 rows of d = 32 db + sigma(lane % 32).
__device__ __forceinline__ int tr_base(int lane) {
  const int h = lane >> 5;
  const int R = (lane >> 2) & 3;
  const int j = lane & 3;
  const int r = 8 * h + R;
  const int ch = 4 * (r & 3) + 2 * ((lane >> 4) & 1) + (j & 1);
  return (r * NCH + ch) * 16 + 8 * (j >> 1);
}

// A operand X^T (rows d = 32 db + sigma(m), k = rows 16 u .. 16 u + 15 of
// the tile) from a transposed-read tile.
__device__ __forceinline__ bf16x8_t tr_frag(const uint4* tile, int base,
                                            int db, int u) {
  const char* p = reinterpret_cast<const char*>(tile) + (base ^ (db << 6)) +
                  16 * u * NCH * 16;
  const i16x4_t x0 = lds_read_tr16(p);
  const i16x4_t x1 = lds_read_tr16(p + 4 * NCH * 16);
  return __builtin_bit_cast(
      bf16x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A operand from a row-layout tile: row sigma(li) of the tile, d chunk
// 8 h + s (k-step s covers d = 8 s .. 8 s + 7 and 64 + 8 s .. 64 + 8 s + 7).
// row_lane gives the lane's chunk offset for k-step 0; step s adds 8 s.
__device__ __forceinline__ int row_lane(int li, int h) {
  const int r = sigma(li);
  return RG * (r >> 3) + 64 * h + (r & 7);
}
__device__ __forceinline__ bf16x8_t row_frag_at(const uint4* tile, int lo,
                                                int s) {
  return as_bf16x8(tile[lo + 8 * s]);
}
__device__ __forceinline__ bf16x8_t row_frag(const uint4* tile, int li, int h,
                                             int s) {
  return row_frag_at(tile, row_lane(li, h), s);
}

// B-operand register fragments of one 128-wide row (query or key) for the
// eight k-steps: lane half h, step s holds d = 64 h + 8 s .. + 7.
__device__ __forceinline__ void load_row_b(const uint16_t* base, int row,
                                           int N, int h, bf16x8_t (&f)[8]) {
  const bool ok = row < N;
  const uint4* src = reinterpret_cast<const uint4*>(
      base + static_cast<int64_t>(ok ? row : 0) * D + 64 * h);
#pragma unroll
  for (int s = 0; s < 8; ++s) f[s] = as_bf16x8(keep_if(src[s], ok));
}

// Store 32 rows x 128 of an O^T-shaped accumulator (row m <-> d = 32 db +
// sigma(m)): lane half h holds d = 32 db + 16 u + 8 h .. + 7 in registers
// 8 u .. 8 u + 7, for the lane's row.
__device__ __forceinline__ void store_rows(uint16_t* dst,
                                           const f32x16_t (&acc)[4],
                                           float mul, int h) {
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const f32x16_t& o = acc[db];
      uint4 w;
      w.x = pack_bf16x2(o[8 * u + 0] * mul, o[8 * u + 1] * mul);
      w.y = pack_bf16x2(o[8 * u + 2] * mul, o[8 * u + 3] * mul);
      w.z = pack_bf16x2(o[8 * u + 4] * mul, o[8 * u + 5] * mul);
      w.w = pack_bf16x2(o[8 * u + 6] * mul, o[8 * u + 7] * mul);
      *reinterpret_cast<uint4*>(dst + 32 * db + 16 * u + 8 * h) = w;
    }
  }
}

// Pack 8 fp32 values (rows 16 u + 8 h .. + 7 of an S-shaped accumulator)
// into the bf16 B operand of k-step u.
__device__ __forceinline__ void pack8(const float (&x)[8], bf16x8_t& b) {
  uint4 w;
  w.x = pack_bf16x2(x[0], x[1]);
  w.y = pack_bf16x2(x[2], x[3]);
  w.z = pack_bf16x2(x[4], x[5]);
  w.w = pack_bf16x2(x[6], x[7]);
  b = as_bf16x8(w);
}

// Pack 16 fp32 values of an S-shaped accumulator (register r <-> tile row
// 16 (r / 8) + 8 h + r % 8) into the two bf16 B operands of k-steps 0, 1.
__device__ __forceinline__ void pack_b(const float (&x)[16],
                                       bf16x8_t (&b)[2]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    uint4 w;
    w.x = pack_bf16x2(x[8 * u + 0], x[8 * u + 1]);
    w.y = pack_bf16x2(x[8 * u + 2], x[8 * u + 3]);
    w.z = pack_bf16x2(x[8 * u + 4], x[8 * u + 5]);
    w.w = pack_bf16x2(x[8 * u + 6], x[8 * u + 7]);
    b[u] = as_bf16x8(w);
  }
}

}  // namespace
}  // namespace fa
