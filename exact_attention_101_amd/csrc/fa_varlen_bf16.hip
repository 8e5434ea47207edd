// Masked forward (bf16, d = 128) for gfx950 (MI355X): variable-length
// batches with narrow sliding windows.  fa_fwd_varlen sends windows bounded
// on both sides and narrower than VARLEN_NARROW keys here; wider and
// unbounded ones run on the pipelined forward kernel (fa_fwd_bf16.hip),
// whose 256-row workgroups would stream W + 256 keys for a window of W.
//
// The FlashAttention-3 summary (GeekNews), section «Comentários no Hacker
// News», asks why FlashAttention is much slower with variable masking and
// how it relates to sliding-window attention.  Here a batch is packed: the
// sequences' rows are concatenated per head (q, o: [H][total_q][d]; k, v:
// [Hkv][total_k][d]; lse: [H][total_q]), cu_seqlens_q / cu_seqlens_k give
// each sequence's first row, and rows of different sequences never meet.
// Within sequence b, with off = Nk_b - Nq_b (bottom-right alignment), query
// i sees key j iff
//     (window_left < 0 or j >= i + off - window_left) and
//     (window_right < 0 or j <= i + off + window_right),
// causal being window_right = 0.  A query that sees no key gets O = 0 and
// LSE = -inf.
//
// Work: one workgroup per (sequence, head, 128 query rows), four waves of
// 32 rows (one lane per row), 32-key tiles of K (row layout) and V
// (transposed-read layout) streamed through LDS by DMA, double-buffered, as
// in the backward's dQ kernel.  Only the tiles the workgroup's rows can see
// are loaded, and a wave skips the arithmetic of tiles its own rows cannot
// see, so the cost follows the window, not the sequence length.  Per tile:
// S^T = K Q^T and O^T += V^T P^T on MFMA in the forward kernel's layouts,
// with an exact online softmax (running maximum and sum over both lane
// halves, rescale of O).  The grid covers the longest sequence; workgroups
// past a shorter sequence's end return at once.
#include "fa_tile32.h"

namespace fa {

namespace {

constexpr float LN2 = 0.69314718055994531f;

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

__global__ void __launch_bounds__(NTHR, 1) varlen_kernel(const VarlenArgs a) {
  __shared__ uint4 K0[ROW_ALLOC];
  __shared__ uint4 K1[ROW_ALLOC];
  __shared__ uint4 V0[TR_SLOTS];
  __shared__ uint4 V1[TR_SLOTS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int h = lane >> 5;

  const int qb = blockIdx.x % a.nqb;
  const int bh = blockIdx.x / a.nqb;
  const int hq = bh % a.H;
  const int b = bh / a.H;
  const int q_beg = a.cu_q[b];
  const int Nq = a.cu_q[b + 1] - q_beg;
  const int k_beg = a.cu_k[b];
  const int Nk = a.cu_k[b + 1] - k_beg;
  // A sequence whose offsets leave the packed tensors is skipped (nothing
  // is read or written for it); so are rows past max_q.
  if (q_beg < 0 || Nq < 0 || q_beg + Nq > a.total_q || k_beg < 0 || Nk < 0 ||
      k_beg + Nk > a.total_k)
    return;
  const int i0 = qb * BLK;
  if (i0 >= Nq) return;                      // whole workgroup, no barrier yet
  const int off = Nk - Nq;
  const int wl = a.left, wr = a.right;
  const int hk = hq / a.group;

  // Visible key range of rows [r0, r1]: [lo, hi] (empty if hi < lo).
  auto key_lo = [&](int r0) { return wl < 0 ? 0 : max(0, r0 + off - wl); };
  auto key_hi = [&](int r1) {
    return wr < 0 ? Nk - 1 : min(Nk - 1, r1 + off + wr);
  };
  const int i1 = min(Nq, i0 + BLK) - 1;
  const int lo = key_lo(i0), hi = key_hi(i1);
  const int t0 = lo / T;
  const int t1 = hi < lo ? t0 : hi / T + 1;  // tiles [t0, t1)
  const int iw0 = i0 + T * wave;
  const int iw1 = min(i1, iw0 + T - 1);
  const bool wave_rows = iw0 <= i1;
  const int wlo = wave_rows ? key_lo(iw0) : 0;
  const int whi = wave_rows ? key_hi(iw1) : -1;

  const int qi = iw0 + li;                   // this lane's query row
  const bool qok = qi < Nq;
  // Keys this lane's row sees: [jlo, jhi] (empty for rows past Nq).
  const int jlo = key_lo(qi);
  const int jhi = qok ? key_hi(qi) : -1;
  const int64_t qrow = static_cast<int64_t>(hq) * a.total_q + q_beg + qi;
  bf16x8_t qf[8];
  load_row_b(static_cast<const uint16_t*>(a.q) +
                 (static_cast<int64_t>(hq) * a.total_q + q_beg) * D,
             qi, Nq, h, qf);

  const int64_t krow0 = static_cast<int64_t>(hk) * a.total_k + k_beg;
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + krow0 * D;
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) + krow0 * D;

  TileCopy cp;
  cp.init(wave, lane);
  const int trb = tr_base(lane);
  auto issue = [&](int t, uint4* kd, uint4* vd) {
    const int r0 = t * T;
    cp.rows(kp, r0, Nk - r0, kd, wave);
    cp.tr(vp, r0, Nk - r0, vd, wave);
  };

  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16_t{};
  float m = -__builtin_inff();
  float l = 0.f;

  // The skip below makes the compiler wait for tile t + 1's copies before
  // the reads of tile t (it cannot tell the stages apart after the branch);
  // with three workgroups per CU that wait costs less than computing
  // masked tiles would.
  auto tile = [&](int t, const uint4* kt, const uint4* vt, uint4* kn,
                  uint4* vn) {
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): tile t landed
    __syncthreads();                         // every wave is done with kn/vn
    if (t + 1 < t1) issue(t + 1, kn, vn);
    const int k0 = t * T;
    if (k0 > whi || k0 + T - 1 < wlo) return;   // no row of this wave sees it
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int f = 0; f < 8; ++f) sc = mfma(row_frag(kt, li, h, f), qf[f], sc);
    // This lane's visible keys [jlo, jhi], relative to its first key of the
    // tile: score x (key k0 + 8 h + kx) is kept iff rlo <= kx <= rhi.
    // When every lane sees all its keys of the tile (kx = 0..7, 16..23), a
    // wave-uniform branch skips the per-key tests.
    const int rlo = jlo - k0 - 8 * h;
    const int rhi = jhi - k0 - 8 * h;
    float mx = -__builtin_inff();
    if (__builtin_amdgcn_ballot_w64(!(rlo <= 0 && rhi >= 23)) == 0) {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        sc[x] *= a.c;
        mx = fmaxf(mx, sc[x]);
      }
    } else {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int kx = 16 * (x >> 3) + (x & 7);
        sc[x] = (kx >= rlo && kx <= rhi) ? sc[x] * a.c : -__builtin_inff();
        mx = fmaxf(mx, sc[x]);
      }
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
    float p[16];
    float sum = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      p[x] = __builtin_amdgcn_exp2f(sc[x] - m_use);
      sum += p[x];
    }
    l += sum;
    bf16x8_t pb[2];
    pack_b(p, pb);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        acc[db] = mfma(tr_frag(vt, trb, db, u), pb[u], acc[db]);
  };

  if (t0 < t1) issue(t0, K0, V0);
  for (int t = t0; t < t1; t += 2) {
    tile(t, K0, V0, K1, V1);
    if (t + 1 < t1) tile(t + 1, K1, V1, K0, V0);
  }

  if (!qok) return;
  const float l_tot = halves_sum(l);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  store_rows(static_cast<uint16_t*>(a.o) + qrow * D, acc, inv, h);
  if (h == 0)
    a.lse[qrow] = (l_tot > 0.f) ? (m + __log2f(l_tot)) * LN2
                                : -__builtin_inff();
}

}  // namespace

hipError_t launch_varlen_bf16(VarlenArgs a, hipStream_t stream) {
  a.nqb = static_cast<int>((static_cast<long long>(a.max_q) + BLK - 1) / BLK);
  const long long grid = static_cast<long long>(a.nqb) * a.H * a.B;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  if (static_cast<long long>(a.total_k) * D * 2 > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(varlen_kernel, dim3((int)grid), dim3(NTHR), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace fa
