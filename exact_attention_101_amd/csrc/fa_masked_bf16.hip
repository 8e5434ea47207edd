// Forward (bf16, d = 128) under an arbitrary visibility mask, for gfx950
// (MI355X).
//
// The FlashAttention-3 summary (GeekNews), section «Comentários no Hacker
// News», reports FlashAttention being much slower with arbitrary masks.
// Here the mask is a bit matrix per (batch, query head), either of which
// may be shared: bit j % 32 of word j / 32 of row i says whether query i
// sees key j.  Scores of hidden keys are -inf, so the softmax runs over the
// visible keys only; a query that sees no key gets O = 0 and LSE = -inf.
//
// Work: one workgroup per (batch, query head, 128 query rows), four waves
// of 32 rows (one lane per row), as in the variable-length kernel.
//   Phase 1: the workgroup ORs its rows' mask words per 32-key tile into a
//   bitmap in LDS (one bit per tile), so the cost of a sparse mask follows
//   the tiles some row of the workgroup sees.
//   Phase 2: the set bits are visited in order; each visited tile's K (row
//   layout) and V (transposed-read layout) arrive by DMA one tile ahead,
//   and each lane's mask word for that tile is loaded with them.  Per tile:
//   S^T = K Q^T, the mask, an exact online softmax (running maximum and sum
//   over both lane halves, rescale of O) and O^T += V^T P^T on MFMA.
#include "fa_tile32.h"

namespace fa {

namespace {

constexpr float LN2 = 0.69314718055994531f;
constexpr int BM_WORDS = MASK_MAX_NK / T / 32;   // tile bitmap, 32 bits/word

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

__global__ void __launch_bounds__(NTHR, 1) masked_kernel(const MaskArgs a) {
  __shared__ uint4 K0[ROW_ALLOC];
  __shared__ uint4 K1[ROW_ALLOC];
  __shared__ uint4 V0[TR_SLOTS];
  __shared__ uint4 V1[TR_SLOTS];
  __shared__ uint32_t bm[BM_WORDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int h = lane >> 5;

  const int qb = blockIdx.x % a.nqb;
  const int bh = blockIdx.x / a.nqb;
  const int hq = bh % a.H;
  const int b = bh / a.H;
  const int hk = hq / a.group;
  const int i0 = qb * BLK;
  const int nrows = min(BLK, a.Nq - i0);
  const int W = a.W;                          // also the number of tiles
  const uint32_t* mp = a.mask + b * a.mask_bs + hq * a.mask_hs;

  // ---- Phase 1: which 32-key tiles does any row of this block see? ----
  for (int t0 = 0; t0 < W; t0 += NTHR) {
    const int t = t0 + tid;
    uint32_t any = 0;
    if (t < W)
      for (int r = 0; r < nrows; ++r)
        any |= mp[static_cast<int64_t>(i0 + r) * W + t];
    const unsigned long long bal = __ballot(any != 0);
    if (lane == 0) {
      bm[(t0 >> 5) + 2 * wave] = static_cast<uint32_t>(bal);
      bm[(t0 >> 5) + 2 * wave + 1] = static_cast<uint32_t>(bal >> 32);
    }
  }
  __syncthreads();
  const int nbw = (W + 31) >> 5;
  // The first tile after t whose bit is set, or W (uniform).
  auto next_tile = [&](int t) {
    int w = (t + 1) >> 5;
    if (w >= nbw) return W;
    uint32_t bits = __builtin_amdgcn_readfirstlane(bm[w]) &
                    (0xFFFFFFFFu << ((t + 1) & 31));
    while (bits == 0) {
      if (++w >= nbw) return W;
      bits = __builtin_amdgcn_readfirstlane(bm[w]);
    }
    return min(W, 32 * w + __builtin_ctz(bits));
  };

  // ---- Phase 2 ----
  const int qi = i0 + T * wave + li;          // this lane's query row
  const bool qok = qi < a.Nq;
  const int64_t qhead = (static_cast<int64_t>(b) * a.H + hq) * a.Nq;
  bf16x8_t qf[8];
  load_row_b(static_cast<const uint16_t*>(a.q) + qhead * D, qi, a.Nq, h, qf);
  const int64_t khead = (static_cast<int64_t>(b) * a.Hkv + hk) * a.Nk;
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + khead * D;
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) + khead * D;
  // This lane's mask row (a valid row for lanes past Nq, whose words are
  // then dropped).
  const uint32_t* mrow = mp + static_cast<int64_t>(qok ? qi : i0) * W;

  TileCopy cp;
  cp.init(wave, lane);
  const int trb = tr_base(lane);
  const int Nk = a.Nk;
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

  // Tile t from (kt, vt) with this lane's mask word mw; tile tn's copies go
  // to (kn, vn) and its mask word to mw_next.
  auto tile = [&](int t, int tn, uint32_t mw, const uint4* kt,
                  const uint4* vt, uint4* kn, uint4* vn, uint32_t& mw_next) {
    __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): tile t landed
    __syncthreads();                         // every wave is done with kn/vn
    if (tn < W) {
      issue(tn, kn, vn);
      mw_next = mrow[tn];
    }
    // Keys past Nk are hidden whatever the mask says (their rows read as
    // zeros): clear their bits once per tile instead of testing every key.
    const int kin = Nk - t * T;
    if (kin < T) mw &= (1u << kin) - 1u;
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int f = 0; f < 8; ++f) sc = mfma(row_frag(kt, li, h, f), qf[f], sc);
    // Lane half h holds keys t T + 16 (x / 8) + 8 h + x % 8.  When every
    // row of the wave sees every key of the tile (dense regions of a mask),
    // the per-key tests are skipped (a wave-uniform branch).  vis: this lane
    // sees some key of the tile.
    bool vis = true;
    if (__builtin_amdgcn_ballot_w64(!(qok && mw == 0xFFFFFFFFu)) == 0) {
#pragma unroll
      for (int x = 0; x < 16; ++x) sc[x] *= a.c;
    } else {
      const uint32_t mh = qok ? (mw >> (8 * h)) : 0u;
      vis = (mh & 0x00FF00FFu) != 0u;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int kx = 16 * (x >> 3) + (x & 7);
        sc[x] = ((mh >> kx) & 1u) ? sc[x] * a.c : -__builtin_inff();
      }
    }
    // P is formed against the m already held (any reference gives the same
    // softmax; a row that has seen no key yet, m = -inf, uses 0).  Only if
    // a lane's sum of p passes 2^8 (or is not finite), or a row sees its
    // first key, does the wave take the exact step: the tile's row maximum,
    // m moved up to it, O and l rescaled, P formed again.  So every p stays
    // in [0, 2^8] and no maximum is computed on the common path.
    float p[16];
    float sum = 0.f;
    {
      const float m_use = (m == -__builtin_inff()) ? 0.f : m;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        p[x] = __builtin_amdgcn_exp2f(sc[x] - m_use);
        sum += p[x];
      }
    }
    const bool bad = !(sum <= 256.0f) || (m == -__builtin_inff() && vis);
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {             // rare
      float mx = -__builtin_inff();
#pragma unroll
      for (int x = 0; x < 16; ++x) mx = fmaxf(mx, sc[x]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m, mx);
      const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
      if (m_new > m) {
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int x = 0; x < 16; ++x) acc[db][x] *= alpha;
      }
      m = m_new;
      sum = 0.f;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        p[x] = __builtin_amdgcn_exp2f(sc[x] - m_use);
        sum += p[x];
      }
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

  int t = next_tile(-1);
  uint32_t mw0 = 0u, mw1 = 0u;
  if (t < W) {
    issue(t, K0, V0);
    mw0 = mrow[t];
  }
  while (t < W) {
    int tn = next_tile(t);
    tile(t, tn, mw0, K0, V0, K1, V1, mw1);
    t = tn;
    if (t >= W) break;
    tn = next_tile(t);
    tile(t, tn, mw1, K1, V1, K0, V0, mw0);
    t = tn;
  }

  if (!qok) return;
  const float l_tot = halves_sum(l);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  store_rows(static_cast<uint16_t*>(a.o) + (qhead + qi) * D, acc, inv, h);
  if (h == 0)
    a.lse[qhead + qi] = (l_tot > 0.f) ? (m + __log2f(l_tot)) * LN2
                                      : -__builtin_inff();
}

}  // namespace

hipError_t launch_masked_bf16(MaskArgs a, hipStream_t stream) {
  a.W = (a.Nk + T - 1) / T;
  a.nqb = static_cast<int>((static_cast<long long>(a.Nq) + BLK - 1) / BLK);
  const long long grid = static_cast<long long>(a.nqb) * a.H * a.B;
  if (grid > 0x7FFFFFFFLL || a.Nk > MASK_MAX_NK)
    return hipErrorInvalidConfiguration;
  if (static_cast<long long>(a.Nk) * D * 2 > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(masked_kernel, dim3((int)grid), dim3(NTHR), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace fa
