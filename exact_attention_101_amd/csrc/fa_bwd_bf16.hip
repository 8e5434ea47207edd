// Attention backward (bf16 in and out, fp32 accumulation) for gfx950
// (MI355X), d = 128.
//
// The pages give the backward pass only in outline: FlashAttention keeps the
// softmax matrix off HBM by recomputing it (FlashAttention-3 summary,
// GeekNews, section «Resumo do FlashAttention»), and the backward pass is
// bound by on-chip shared-memory traffic rather than the matrix units
// (FlashAttention-4 page, smntcn.com, paragraph 2).  The gradients are those
// of O = softmax(scale Q K^T [+ causal mask]) V for a given dO:
//     P = exp(scale Q K^T - LSE)     (recomputed from the forward's LSE)
//     dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i,  dS = P * (dP - D)
//     dQ = scale dS K,  dK = scale dS^T Q
//
// Three launches, no atomics, deterministic:
//   * bwd_prep_kernel: ws[i] = {LSE_i log2(e), D_i} for every query row.
//   * bwd_dq_kernel: one lane per query, as in the forward kernel; 32-key
//     tiles of K and V stream through LDS.  S^T = K Q^T and dP^T = V dO^T on
//     MFMA (K and V rows in the forward's sigma order, Q^T and dO^T held as
//     B operands in registers), dS^T in the layout of the forward's P, and
//     dQ^T += K^T dS^T with K^T read by the transposing LDS read, exactly
//     the forward's O^T += V^T P^T.
//   * bwd_dkdv_kernel: one lane per key; 32-query tiles of Q and dO (and
//     their ws entries) stream through LDS for every query head of the KV
//     head's group.  S = Q K^T and dP = dO V^T with K^T and V^T held in
//     registers, then dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T
//     from transposing reads.
//
// LDS tile layouts and copy plans: fa_tile32.h.
#include "fa_tile32.h"

namespace fa {

namespace {

// ---- ws[i] = {LSE_i log2(e), dO_i . O_i}: 16 lanes per row ----
__global__ void __launch_bounds__(256) bwd_prep_kernel(const BwdArgs a,
                                                       long long rows) {
  const long long row = static_cast<long long>(blockIdx.x) * 16 +
                        (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const uint4 x = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.o) + row * D)[c];
    const uint4 y = reinterpret_cast<const uint4*>(
        static_cast<const uint16_t*>(a.dout) + row * D)[c];
    const bf16x8_t xo = as_bf16x8(x), yo = as_bf16x8(y);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      acc = fmaf(static_cast<float>(xo[i]), static_cast<float>(yo[i]), acc);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (row < rows && c == 0) {
    a.ws[2 * row] = a.lse[row] * LOG2E;
    a.ws[2 * row + 1] = acc;
  }
}

// ---- dQ: one lane per query ----
template <bool CAUSAL>
__global__ void __launch_bounds__(NTHR, 1) bwd_dq_kernel(const BwdArgs a) {
  // One array per stage and operand: every LDS read then names the array
  // it reads, so the compiler need not wait for copies into the other stage.
  __shared__ uint4 Kr0[ROW_ALLOC], Kr1[ROW_ALLOC];
  __shared__ uint4 Kt0[TR_SLOTS], Kt1[TR_SLOTS];
  __shared__ uint4 Vr0[ROW_ALLOC], Vr1[ROW_ALLOC];

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
  const int q0 = qb * BLK;
  const int qw0 = q0 + T * wave;
  const int qrow = qw0 + li;

  const int64_t qhead = (static_cast<int64_t>(b) * a.H + hq) * N;
  const int64_t khead = (static_cast<int64_t>(b) * a.Hkv + hk) * N;
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + khead * D;
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) + khead * D;

  bf16x8_t qf[8], of[8];
  load_row_b(static_cast<const uint16_t*>(a.q) + qhead * D, qrow, N, h, qf);
  load_row_b(static_cast<const uint16_t*>(a.dout) + qhead * D, qrow, N, h,
             of);
  const bool qok = qrow < N;
  const float lse2 = qok ? a.ws[2 * (qhead + qrow)] : 0.f;
  const float dq_row = qok ? a.ws[2 * (qhead + qrow) + 1] : 0.f;

  TileCopy cp;
  cp.init(wave, lane);
  const int trb = tr_base(lane);

  const int kv_end = CAUSAL ? min(N, q0 + BLK) : N;
  const int ntiles = (kv_end + T - 1) / T;
  auto issue = [&](int t, uint4* kr, uint4* kt, uint4* vr) {
    const int r0 = t * T;
    cp.rows(kp, r0, kv_end - r0, kr, wave);
    cp.tr(kp, r0, kv_end - r0, kt, wave);
    cp.rows(vp, r0, kv_end - r0, vr, wave);
  };

  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16_t{};

  // Key tile t from (kr, kt, vr); tile t + 1's copies go to (nkr, nkt, nvr).
  // Waves whose rows see none of the tile's keys still run it, fully
  // masked (p = 0): a branch here would make the compiler wait for the
  // copies just issued before every LDS read.
  auto step = [&](int t, const uint4* kr, const uint4* kt, const uint4* vr,
                  uint4* nkr, uint4* nkt, uint4* nvr) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this tile has landed
    __syncthreads();                      // and every wave is done with n*
    if (t + 1 < ntiles) issue(t + 1, nkr, nkt, nvr);
    const int k0 = t * T;
    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
    for (int f = 0; f < 8; ++f) s = mfma(row_frag(kr, li, h, f), qf[f], s);
#pragma unroll
    for (int f = 0; f < 8; ++f) dp = mfma(row_frag(vr, li, h, f), of[f], dp);
    float ds[16];
    if (k0 + T <= N && (!CAUSAL || k0 + T - 1 <= qw0)) {
      // Every key of the tile is visible to every row of the wave (the
      // test is wave-uniform).  Lanes of rows past N see finite values
      // (zero Q and dO, zero {LSE, D}) and their dQ is never stored.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[r], a.c, -lse2));
        ds[r] = p * (dp[r] - dq_row);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 16 * (r >> 3) + 8 * h + (r & 7);
        const bool ok = qok && key < N && (!CAUSAL || key <= qrow);
        // exp2(-inf) = 0 masks without a branch.
        const float p = __builtin_amdgcn_exp2f(
            ok ? fmaf(s[r], a.c, -lse2) : -__builtin_inff());
        ds[r] = p * (dp[r] - dq_row);
      }
    }
    bf16x8_t dsb[2];
    pack_b(ds, dsb);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        acc[db] = mfma(tr_frag(kt, trb, db, u), dsb[u], acc[db]);
  };

  issue(0, Kr0, Kt0, Vr0);
  for (int t = 0; t < ntiles; t += 2) {
    step(t, Kr0, Kt0, Vr0, Kr1, Kt1, Vr1);
    if (t + 1 < ntiles) step(t + 1, Kr1, Kt1, Vr1, Kr0, Kt0, Vr0);
  }

  if (qok) {
    uint16_t* dst =
        static_cast<uint16_t*>(a.dq) + (qhead + qrow) * static_cast<int64_t>(D);
    store_rows(dst, acc, a.scale, h);
  }
}

// ---- dK, dV: one lane per key ----
// Two workgroups per CU (two waves per SIMD), each with 256 registers.
template <bool CAUSAL>
__global__ void __launch_bounds__(NTHR, 2) bwd_dkdv_kernel(const BwdArgs a) {
  // One array per stage and operand (see the dQ kernel).
  __shared__ uint4 Qr0[ROW_ALLOC], Qr1[ROW_ALLOC];
  __shared__ uint4 Qt0[TR_SLOTS], Qt1[TR_SLOTS];
  __shared__ uint4 Or0[ROW_ALLOC], Or1[ROW_ALLOC];   // dO, row layout
  __shared__ uint4 Ot0[TR_SLOTS], Ot1[TR_SLOTS];     // dO, transposed
  __shared__ float Ws0[2 * T], Ws1[2 * T];  // {LSE log2(e), D} of the rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int h = lane >> 5;

  // Causal: key-block-major order, every head's block 0, then every head's
  // block 1, and so on.  Block 0 meets every query and the last block the
  // fewest, so the longest work is dispatched first and the tail is short;
  // and since workgroups go to the XCDs in turn, all blocks of one head
  // share an XCD and its L2 when B * Hkv is a multiple of 8.  Non-causal
  // blocks are equal and head-major order measures slightly faster.
  const int unit = blockIdx.x;
  const int nbhk = a.B * a.Hkv;
  const int kb = CAUSAL ? unit / nbhk : unit % a.nkb;
  const int bhk = CAUSAL ? unit % nbhk : unit / a.nkb;
  const int b = bhk / a.Hkv;
  const int hk = bhk % a.Hkv;
  const int N = a.N;
  const int k0 = kb * BLK;
  const int kw0 = k0 + T * wave;
  const int key = kw0 + li;

  const int64_t khead = (static_cast<int64_t>(b) * a.Hkv + hk) * N;
  bf16x8_t kf[8], vf[8];
  load_row_b(static_cast<const uint16_t*>(a.k) + khead * D, key, N, h, kf);
  load_row_b(static_cast<const uint16_t*>(a.v) + khead * D, key, N, h, vf);

  TileCopy cp;
  cp.init(wave, lane);
  const int trb = tr_base(lane);
  const int rlo = row_lane(li, h);

  // Query tiles: every query head of the group, from the first tile that
  // holds a query >= k0 (causal) or 0.  Causal blocks walk each head's
  // tiles from the last one down, so that the blocks of one head, which
  // start together, read the same query tiles at about the same time.
  const int t0 = CAUSAL ? k0 / T : 0;
  const int ntq = (N + T - 1) / T;
  const int per_head = ntq - t0;
  const int nsteps = per_head * a.group;
  auto tile_of = [&](int step) {
    const int i = step % per_head;
    return CAUSAL ? ntq - 1 - i : i;
  };
  struct Stage {
    uint4* qr;
    uint4* qt;
    uint4* orow;
    uint4* ot;
    float* ws;
  };
  const Stage s0{Qr0, Qt0, Or0, Ot0, Ws0};
  const Stage s1{Qr1, Qt1, Or1, Ot1, Ws1};

  auto issue = [&](int step, const Stage& d) {
    const int hq = hk * a.group + step / per_head;
    const int t = tile_of(step);
    const int64_t qhead = (static_cast<int64_t>(b) * a.H + hq) * N;
    const int r0 = t * T;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qhead * D;
    const uint16_t* op = static_cast<const uint16_t*>(a.dout) + qhead * D;
    cp.rows(qp, r0, N - r0, d.qr, wave);
    cp.tr(qp, r0, N - r0, d.qt, wave);
    cp.rows(op, r0, N - r0, d.orow, wave);
    cp.tr(op, r0, N - r0, d.ot, wave);
    if (wave == 0) {
      const auto rw = rows_rsrc(a.ws + 2 * qhead, r0, N - r0, 8);
      copy4(rw, d.ws, 4u * lane);
    }
  };

  f32x16_t dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dk[i] = f32x16_t{};
    dv[i] = f32x16_t{};
  }

  // Query tile `step` from c; the next one's copies go to n.  Waves whose
  // keys no query of the tile sees (causal) still run it, fully masked.
  auto run = [&](int step, const Stage& c, const Stage& n) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (step + 1 < nsteps) issue(step + 1, n);
    const int qt0 = tile_of(step) * T;
    // LDS read addresses (the four d-block variants of the transposed one,
    // the row-layout ones of the two tiles, the {LSE, D} one) are formed
    // here from opaque copies the compiler cannot hoist, so that they hold
    // registers only while used: the loop needs every register it has.
    int tb = trb, ro = rlo, wo = 16 * h;
    asm volatile("" : "+v"(tb), "+v"(ro), "+v"(wo));
    f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
    for (int f = 0; f < 8; ++f) s = mfma(row_frag_at(c.qr, ro, f), kf[f], s);
#pragma unroll
    for (int f = 0; f < 8; ++f)
      dp = mfma(row_frag_at(c.orow, ro, f), vf[f], dp);
    // Rows 16 u + 8 h .. + 7 of the tile (k-step u of the dV / dK MFMAs):
    // their {LSE log2 e, D} pairs are 16 consecutive floats.  Each half is
    // packed and fed to the matrix core as soon as it is formed.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float4* wp =
          reinterpret_cast<const float4*>(&c.ws[32 * u + wo]);
      float w[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = wp[i];
        w[4 * i] = x.x; w[4 * i + 1] = x.y; w[4 * i + 2] = x.z;
        w[4 * i + 3] = x.w;
      }
      // Only the causal mask is applied.  Query rows past N arrive as
      // zeros (Q, dO and their {LSE, D} pair), so their p = 1 meets
      // dO = 0 and dP - D = 0 and adds nothing; keys past N are not stored.
      float p[8], ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * u + j;
        const float x = fmaf(s[r], a.c, -w[2 * j]);
        // exp2(-inf) = 0 masks without a branch.
        p[j] = __builtin_amdgcn_exp2f(
            (!CAUSAL || key <= qt0 + 16 * u + 8 * h + j) ? x
                                                         : -__builtin_inff());
        ds[j] = p[j] * (dp[r] - w[2 * j + 1]);
      }
      bf16x8_t pb, dsb;
      pack8(p, pb);
      pack8(ds, dsb);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dv[db] = mfma(tr_frag(c.ot, tb, db, u), pb, dv[db]);
        dk[db] = mfma(tr_frag(c.qt, tb, db, u), dsb, dk[db]);
      }
    }
  };

  if (nsteps > 0) issue(0, s0);
  for (int step = 0; step < nsteps; step += 2) {
    run(step, s0, s1);
    if (step + 1 < nsteps) run(step + 1, s1, s0);
  }

  // The lane's key is formed again from the lane count rather than held
  // across the loop, which needs every vector register (held, it was
  // spilled to memory).
  const int elane =
      __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int ekey = kw0 + (elane & 31);
  if (ekey < N) {
    const int64_t off = (khead + ekey) * static_cast<int64_t>(D);
    store_rows(static_cast<uint16_t*>(a.dk) + off, dk, a.scale, elane >> 5);
    store_rows(static_cast<uint16_t*>(a.dv) + off, dv, 1.f, elane >> 5);
  }
}

}  // namespace

hipError_t launch_bwd_bf16(BwdArgs a, bool causal, hipStream_t stream) {
  const long long rows = static_cast<long long>(a.B) * a.H * a.N;
  const long long prep_grid = (rows + 15) / 16;
  a.nqb = static_cast<int>((static_cast<long long>(a.N) + BLK - 1) / BLK);
  a.nkb = a.nqb;
  const long long dq_grid = static_cast<long long>(a.B) * a.H * a.nqb;
  const long long kv_grid = static_cast<long long>(a.B) * a.Hkv * a.nkb;
  if (prep_grid > 0x7FFFFFFFLL || dq_grid > 0x7FFFFFFFLL ||
      kv_grid > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  // Per-head byte ranges are addressed by 32-bit buffer offsets.
  if (static_cast<long long>(a.N) * D * 2 > 0x7FFFFFFFLL)
    return hipErrorInvalidConfiguration;
  const int bh = a.B * a.H;
  a.xcd_chunk = causal ? (bh % 8 == 0) : (dq_grid % 8 == 0);
  hipLaunchKernelGGL(bwd_prep_kernel, dim3((int)prep_grid), dim3(256), 0,
                     stream, a, rows);
  if (causal) {
    hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3((int)dq_grid), dim3(NTHR), 0,
                       stream, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<true>, dim3((int)kv_grid), dim3(NTHR),
                       0, stream, a);
  } else {
    hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3((int)dq_grid), dim3(NTHR),
                       0, stream, a);
    hipLaunchKernelGGL(bwd_dkdv_kernel<false>, dim3((int)kv_grid),
                       dim3(NTHR), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace fa
