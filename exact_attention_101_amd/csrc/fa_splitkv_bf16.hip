// Split-KV attention forward (bf16, d = 128) for decode-shaped work on
// gfx950 (MI355X): Nq queries (a few) against Nk keys (many).
//
// The pages motivate this only as long-context processing (FlashAttention-3
// summary, GeekNews, sections «Importância do Attention» and «Melhorias de
// desempenho do FlashAttention-3»).  With few queries per head the forward
// kernel's 256-row blocks would sit nearly empty and a handful of
// workgroups would stream all of K and V, so the key range is split instead:
//
//   * splitkv_kernel: one wave = one work item (batch b, KV head hk, block of
//     32 rows, split s).  The rows of a KV head are its group's (query,
//     head) pairs, r = i * group + g, so K and V are read once for all the
//     query heads that share them.  The wave streams its split's 32-key
//     tiles of K and V through its own double-buffered LDS (DMA, no
//     barriers), computes S^T = K Q^T and O^T += V^T P^T on MFMA exactly as
//     the forward kernel lays them out (K rows in sigma order, V^T by
//     transposing reads), with a plain online softmax (running maximum,
//     running sum, rescale of O), and writes its normalised partial O_s
//     (fp32) and LSE_s (log2 units) to the workspace.
//   * splitkv_merge_kernel: per query row (one block of 256 threads over
//     the splits), LSE = log2 sum_s 2^LSE_s and
//     O = sum_s 2^(LSE_s - LSE) O_s (splits that saw no key have LSE_s =
//     -inf and weight 0), written as bf16 O and natural-log LSE.
//
// Causal masks use bottom-right alignment: query i sees key j iff
// j <= i + Nk - Nq.  Key tiles of a split past its rows' last visible key
// are not loaded.
//
// The kernel is bound by HBM: per key it reads 512 bytes of K and V and
// does 4 d FLOPs per row, so up to 32 rows it stays far below the MFMA
// ridge.
#include <mutex>

#include "fa_common.h"

namespace fa {

// Scratch of the entry point that allocates nothing (fa_fwd_splitkv_noalloc):
// the splits' partial outputs and LSEs, SPLITKV_SCRATCH_FLOATS floats that
// every GPU the library runs on holds until the process ends.  In host code
// `scratch` names a host-side stand-in, not a device address: the device
// address is taken once per device with hipGetSymbolAddress (with that
// device current) and only that address is passed to kernels.  All calls on
// one GPU share its copy; calls that overlap on one GPU race.  Nothing in it
// needs clearing: every (split, row) entry the merge reads is written first.
static __device__ __align__(256) float scratch[SPLITKV_SCRATCH_FLOATS];

namespace {

constexpr int D = 128;
constexpr int NCH = D / 8;            // 16-byte chunks per row
constexpr int T = 32;                 // keys per tile
// Waves (independent items) per block: 5 x 32 KB of double-buffered K / V
// tiles fill the 160 KB of LDS, so each CU keeps 5 tiles of K and V (80 KB)
// in flight from HBM (4 waves: 64 KB, 6-14% slower on decode shapes).
constexpr int NW = 5;
constexpr int TILE = T * NCH;         // chunks per tile (512)
constexpr float LN2 = 0.69314718055994531f;

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

// v_permlane32_swap of x with itself returns, in every lane, the value of
// the low lane half (r[0]) and of the high lane half (r[1]) for the same
// lane % 32: combining both gives the row's value over both halves.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t rsrc,
                                       const void* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)(dst), 16, voffset, 0, 0,
      0);
}

// Physical chunk of (row r, logical chunk c) in a K tile: the chunk index is
// XOR-ed with r % 16, so the 16 rows that one read phase takes at the same
// logical chunk (rows sigma(li), a permutation of each group of 16) sit in
// 16 different 16-byte bank groups of the 256-byte bank row.
__device__ __forceinline__ int kswz(int r, int c) {
  return r * NCH + (c ^ (r & 15));
}

template <bool CAUSAL>
__global__ void __launch_bounds__(64 * NW, 1)
splitkv_kernel(const SplitArgs a) {
  // Two stages as separate arrays, so the compiler sees that the copies
  // into one stage do not feed the reads of the other.
  __shared__ uint4 K0[NW][TILE];
  __shared__ uint4 K1[NW][TILE];
  __shared__ uint4 V0[NW][TILE];
  __shared__ uint4 V1[NW][TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 31;
  const int h = lane >> 5;

  const long long item = static_cast<long long>(blockIdx.x) * NW + wave;
  if (item >= a.items) return;               // whole wave leaves; no barriers
  const int s = static_cast<int>(item % a.splits);
  const long long rest = item / a.splits;
  const int rb = static_cast<int>(rest % a.nrb);
  const int bhk = static_cast<int>(rest / a.nrb);
  const int b = bhk / a.Hkv;
  const int hk = bhk % a.Hkv;
  const int Nq = a.Nq, Nk = a.Nk;
  const int rows = Nq * a.group;             // rows of this KV head

  // This lane's row (both lane halves hold the same row).
  const int r = rb * T + li;
  const bool rok = r < rows;
  const int qi = rok ? r / a.group : 0;
  const int hq = hk * a.group + (rok ? r % a.group : 0);
  const int64_t qrow = (static_cast<int64_t>(b) * a.H + hq) * Nq + qi;

  // Q^T as the B operand: lane half h, k-step t holds d = 64 h + 8 t .. + 7.
  bf16x8_t qf[8];
  {
    const uint4* src = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.q) + qrow * D + 64 * h);
#pragma unroll
    for (int t = 0; t < 8; ++t) qf[t] = as_bf16x8(keep_if(src[t], rok));
  }

  // Key tiles of split s: [kb0, kb1), clipped to the last key any row of
  // the block can see.
  const int nkb = (Nk + T - 1) / T;
  int kb0 = static_cast<int>(static_cast<long long>(s) * nkb / a.splits);
  int kb1 = static_cast<int>(static_cast<long long>(s + 1) * nkb / a.splits);
  const int off = Nk - Nq;                   // bottom-right causal offset
  // This lane's last visible key (-1: none; rows past the block see none).
  const int jhi = !rok ? -1 : (CAUSAL ? min(Nk - 1, qi + off) : Nk - 1);
  if (CAUSAL) {
    const int r_last = min(rows, rb * T + T) - 1;
    const int last_key = r_last / a.group + off;   // max over the block
    kb1 = min(kb1, last_key < 0 ? 0 : last_key / T + 1);
  }

  const int64_t khead = (static_cast<int64_t>(b) * a.Hkv + hk) * Nk;
  const char* kp = static_cast<const char*>(a.k) + khead * D * 2;
  const char* vp = static_cast<const char*>(a.v) + khead * D * 2;

  // Copy j of a tile: lane writes chunk 64 j + lane = (row, physical p),
  // whose logical chunk is the same XOR applied again.  V: the 64-byte
  // segment index is XOR-ed with row % 4, so the 4 rows of one transposing
  // read hit 4 different bank groups; K: kswz's chunk XOR.  Each copy reads
  // 4 whole rows.
  uint32_t coff[TILE / 64], kcoff[TILE / 64];
#pragma unroll
  for (int j = 0; j < TILE / 64; ++j) {
    const int slot = 64 * j + lane;
    const int rr = slot / NCH, p = slot % NCH;
    const int c = (((p >> 2) ^ (rr & 3)) << 2) | (p & 3);
    coff[j] = static_cast<uint32_t>(rr * D * 2 + c * 16);
    kcoff[j] = static_cast<uint32_t>(rr * D * 2 + (p ^ (rr & 15)) * 16);
  }
  auto issue = [&](int kb, uint4* kd, uint4* vd) {
    const int k0 = kb * T;
    const int nrows = max(Nk - k0, 0);
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(kp + static_cast<int64_t>(k0) * D * 2), 0,
        nrows * D * 2, 0x00020000);
    const auto rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(vp + static_cast<int64_t>(k0) * D * 2), 0,
        nrows * D * 2, 0x00020000);
#pragma unroll
    for (int j = 0; j < TILE / 64; ++j) {
      copy16(rk, kd + 64 * j, kcoff[j]);
      copy16(rv, vd + 64 * j, coff[j]);
    }
  };

  // Transposed V read base (the forward kernel's V reads): lane 16 g + 4 R
  // + j reads row 8 h + R at d = 16 (g % 2) + 8 (j % 2) + 4 (j / 2); the
  // output lane holds 4 keys of d = 32 db + sigma(lane % 32).
  int trb;
  {
    const int R = (lane >> 2) & 3, j = lane & 3;
    const int rr = 8 * h + R;
    const int ch = 4 * (rr & 3) + 2 * ((lane >> 4) & 1) + (j & 1);
    trb = (rr * NCH + ch) * 16 + 8 * (j >> 1);
  }

  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16_t{};
  float m = -__builtin_inff();               // running max, log2 units
  float l = 0.f;                             // this half's running sum

  // One 32-key tile: its copies landed in (kt, vt); the next tile's go
  // into (kn, vn).
  auto tile = [&](int kb, const uint4* kt, const uint4* vt, uint4* kn,
                  uint4* vn) {
    // The tile's copies have landed, and this wave's reads of the other
    // stage (the previous tile) are done before new copies overwrite it.
    __builtin_amdgcn_s_waitcnt(0x0070);      // vmcnt(0), lgkmcnt(0)
    if (kb + 1 < kb1) issue(kb + 1, kn, vn);
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int t = 0; t < 8; ++t)
      sc = mfma(as_bf16x8(kt[kswz(sigma(li), 8 * h + t)]), qf[t], sc);
    // Scale, mask; lane half h holds keys 16 (x / 8) + 8 h + x % 8.
    // Score x is key kb T + 8 h + kx: kept iff kx <= rhi (this lane's last
    // visible key, relative to its first key of the tile).
    const int rhi = jhi - kb * T - 8 * h;
    float mx = -__builtin_inff();
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int kx = 16 * (x >> 3) + (x & 7);
      sc[x] = (kx <= rhi) ? sc[x] * a.c : -__builtin_inff();
      mx = fmaxf(mx, sc[x]);
    }
    mx = halves_max(mx);
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    // O and l are rescaled only when some row's maximum grew in this tile
    // (alpha = 1 for every row otherwise); the test is wave-uniform.
    if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int x = 0; x < 16; ++x) acc[db][x] *= alpha;
    }
    m = m_new;
    float pr[16];
    float sum = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      pr[x] = __builtin_amdgcn_exp2f(sc[x] - m_use);
      sum += pr[x];
    }
    l += sum;
    bf16x8_t pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint4 w;
      w.x = pack_bf16x2(pr[8 * u + 0], pr[8 * u + 1]);
      w.y = pack_bf16x2(pr[8 * u + 2], pr[8 * u + 3]);
      w.z = pack_bf16x2(pr[8 * u + 4], pr[8 * u + 5]);
      w.w = pack_bf16x2(pr[8 * u + 6], pr[8 * u + 7]);
      pb[u] = as_bf16x8(w);
    }
    const char* vb = reinterpret_cast<const char*>(vt);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const char* p = vb + (trb ^ (db << 6)) + 16 * u * NCH * 16;
        const i16x4_t x0 = lds_read_tr16(p);
        const i16x4_t x1 = lds_read_tr16(p + 4 * NCH * 16);
        const bf16x8_t v8 = __builtin_bit_cast(
            bf16x8_t,
            __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = mfma(v8, pb[u], acc[db]);
      }
  };

  if (kb0 < kb1) issue(kb0, K0[wave], V0[wave]);
  for (int kb = kb0; kb < kb1; kb += 2) {
    tile(kb, K0[wave], V0[wave], K1[wave], V1[wave]);
    if (kb + 1 < kb1) tile(kb + 1, K1[wave], V1[wave], K0[wave], V0[wave]);
  }

  if (!rok) return;
  const float l_tot = halves_sum(l);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const int64_t prow = static_cast<int64_t>(s) * a.rows_total + qrow;
  float* op = a.ws_o + prow * D;
  // Accumulator row m <-> d = 32 db + sigma(m): lane half h holds
  // d = 32 db + 16 u + 8 h .. + 7 in registers 8 u .. 8 u + 7.
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float4* dst = reinterpret_cast<float4*>(op + 32 * db + 16 * u + 8 * h);
      dst[0] = make_float4(acc[db][8 * u] * inv, acc[db][8 * u + 1] * inv,
                           acc[db][8 * u + 2] * inv, acc[db][8 * u + 3] * inv);
      dst[1] = make_float4(acc[db][8 * u + 4] * inv, acc[db][8 * u + 5] * inv,
                           acc[db][8 * u + 6] * inv, acc[db][8 * u + 7] * inv);
    }
  if (h == 0)
    a.ws_lse[prow] = (l_tot > 0.f) ? m + __log2f(l_tot) : -__builtin_inff();
}

// One block of 256 threads per query row.  The row's splits are spread
// over all threads for the log-sum-exp, and over 4 groups of 64 threads
// (2 values of d each) for the weighted sum of the partial outputs, so rows
// with many splits are not merged by a serial loop.
__global__ void __launch_bounds__(256) splitkv_merge_kernel(const SplitArgs a) {
  __shared__ float red[256];
  __shared__ float2 part[3][64];
  const long long row = blockIdx.x;
  const int t = threadIdx.x;
  const int S = a.splits;
  const float* lse_s = a.ws_lse + row;                 // stride rows_total
  const long long stride = a.rows_total;

  float mx = -__builtin_inff();
  for (int s = t; s < S; s += 256) mx = fmaxf(mx, lse_s[s * stride]);
  red[t] = mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] = fmaxf(red[t], red[t + w]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float z = 0.f;
  if (mx != -__builtin_inff())
    for (int s = t; s < S; s += 256)
      z += __builtin_amdgcn_exp2f(lse_s[s * stride] - mx);
  red[t] = z;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  const float lse2 = (mx == -__builtin_inff()) ? -__builtin_inff()
                                               : mx + __log2f(red[0]);

  const int dp = t & 63;                               // d = 2 dp, 2 dp + 1
  const int g = t >> 6;                                // split group
  float2 o = make_float2(0.f, 0.f);
  if (lse2 != -__builtin_inff()) {
    // Unrolled so that several splits' loads are in flight at once.
#pragma unroll 8
    for (int s = g; s < S; s += 4) {
      const float w = __builtin_amdgcn_exp2f(lse_s[s * stride] - lse2);
      const float2 x = reinterpret_cast<const float2*>(
          a.ws_o + (static_cast<int64_t>(s) * stride + row) * D)[dp];
      o.x = fmaf(w, x.x, o.x);
      o.y = fmaf(w, x.y, o.y);
    }
  }
  if (g > 0) part[g - 1][dp] = o;
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      o.x += part[i][dp].x;
      o.y += part[i][dp].y;
    }
    reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.o) + row * D)[dp] =
        pack_bf16x2(o.x, o.y);
    if (dp == 0) a.lse[row] = lse2 * LN2;
  }
}

}  // namespace

int splitkv_auto_splits(int B, int H, int Hkv, int Nq, int Nk) {
  const long long rows = static_cast<long long>(Nq) * (H / Hkv);
  const long long nrb = (rows + T - 1) / T;
  // B * Hkv * nrb can pass 2^63 for sizes at the int limits; only whether it
  // reaches 1024 matters.
  const long long bk = static_cast<long long>(B) * Hkv;
  const long long units = (bk >= 1024 || nrb >= 1024) ? 1024 : bk * nrb;
  const long long nkb = (static_cast<long long>(Nk) + T - 1) / T;
  // About 1024 waves, one round at this kernel's 5 waves per CU, each split
  // at least 4 tiles.  Measured on decode shapes against 1280, 2048 and 2560
  // waves: best or tied everywhere (two rounds leave a tail, and split
  // counts that are not powers of two cut the key range unevenly).
  long long s = (1024 + units - 1) / units;
  const long long cap = nkb / 4 > 1 ? nkb / 4 : 1;
  if (s > cap) s = cap;
  if (s > SPLITKV_MAX_SPLITS) s = SPLITKV_MAX_SPLITS;
  return static_cast<int>(s < 1 ? 1 : s);
}

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex scratch_mu;
float* scratch_ptr[SCRATCH_MAX_DEVICES] = {};
}  // namespace

// Device address of this device's scratch (the current device's), set up on
// the first call on each device.
hipError_t splitkv_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_splitkv_bf16(SplitArgs a, bool causal, hipStream_t stream) {
  a.group = a.H / a.Hkv;
  const long long rows = static_cast<long long>(a.Nq) * a.group;
  a.nrb = static_cast<int>((rows + T - 1) / T);
  a.items = static_cast<long long>(a.B) * a.Hkv * a.nrb * a.splits;
  a.rows_total = static_cast<long long>(a.B) * a.H * a.Nq;
  const long long grid = (a.items + NW - 1) / NW;
  const long long mgrid = a.rows_total;
  if (grid > 0x7FFFFFFFLL || mgrid > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  if (static_cast<long long>(a.Nk) * D * 2 > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  if (causal) {
    hipLaunchKernelGGL(splitkv_kernel<true>, dim3((int)grid), dim3(64 * NW),
                       0, stream, a);
  } else {
    hipLaunchKernelGGL(splitkv_kernel<false>, dim3((int)grid), dim3(64 * NW),
                       0, stream, a);
  }
  hipLaunchKernelGGL(splitkv_merge_kernel, dim3((int)mgrid), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace fa
