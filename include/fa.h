/*
 * fa.h -- C ABI of the MI355X (gfx950) FlashAttention forward library
 * (libfa.so).
 *
 * The operation.  Exact scaled-dot-product attention,
 *     O = softmax(scale * Q K^T [+ causal mask]) V,
 * softmax over keys, computed the FlashAttention way: Q is split into row
 * blocks, the K/V blocks stream past each one through on-chip memory, and an
 * online softmax keeps a running row maximum, a running denominator and a
 * running output that is rescaled whenever the maximum grows, so the N x N
 * score matrix never reaches device memory.  Sources: the FlashAttention v1
 * post (DeepSchool #630), sections «Проблема базового attention» (the
 * operation and the cost of materialising Q K^T), «Тайлинг (Tiling)» (row
 * blocks of Q against streamed K/V blocks), «Онлайн-Softmax» (running max,
 * running denominator, rescale of the partial output) and «Итог» (linear
 * memory); the FlashAttention-3 summary (GeekNews), section «Resumo do
 * FlashAttention» (the attention matrix is never written out).  Besides O
 * the forward writes the per-row natural-log log-sum-exp LSE of the scaled,
 * masked scores, the only other output.
 *
 * Conventions shared by every entry point:
 *   - Device pointers are HIP device allocations owned by the caller.  The
 *     library never allocates or frees device memory and never synchronises
 *     the device; calls are thread-safe.  The only global state is the
 *     fixed per-device scratch of fa_fwd_splitkv_noalloc (see there) and a
 *     per-device cache of the compute-unit count (read once, used to size
 *     the persistent launch of the dense non-causal forward).
 *   - Layouts are dense row-major:  q, o: [B][H][N][d];  k, v: [B][Hkv][N][d];
 *     lse: [B][H][N] (float, natural log).  All offsets are 64-bit.
 *   - Grouped-query attention: H must be a multiple of Hkv; query head h
 *     reads key/value head h / (H / Hkv).
 *   - causal != 0 hides key j from query i when j > i.
 *   - Work is only enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream).  Errors raised while a kernel runs surface at the caller's
 *     next synchronisation.
 *   - Outputs are fully overwritten; inputs are never written.  Outputs must
 *     not alias inputs.
 *   - Return value: an fa_status_t.  Arguments are checked in this order and
 *     the first failure is returned before anything is enqueued:
 *       FA_ERR_INVALID_ARGUMENT  null pointer, B/H/Hkv/N/d <= 0, H % Hkv != 0,
 *                                non-finite scale, sizes whose element
 *                                counts overflow 64 bits;
 *       FA_ERR_UNSUPPORTED       d not supported by the kernel family, or an
 *                                unknown dtype;
 *       FA_ERR_MISALIGNED        a tensor pointer not 16-byte aligned;
 *       FA_ERR_HIP               the launch failed (fa_last_hip_error() gives
 *                                the hipError_t);
 *       FA_ERR_WORKSPACE         (fa_fwd_splitkv_noalloc only) the sizes do
 *                                not fit in its fixed scratch.
 */
#ifndef FA_H_
#define FA_H_

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_DTYPE_BF16 = 0,      /* q, k, v, o: bfloat16 */
  FA_DTYPE_FP8_E4M3 = 1   /* q, k, v: OCP e4m3 ("e4m3fn") codes; o: bfloat16 */
} fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARGUMENT = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_MISALIGNED = 3,
  FA_ERR_HIP = 4,
  FA_ERR_WORKSPACE = 5
} fa_status_t;

/*
 * fa_fwd -- attention forward.
 *   q, k, v  device, dtype as below, layouts as above (read only).
 *   o        device, bfloat16 [B][H][N][d] (written).
 *   lse      device, float [B][H][N] (written): ln sum_j exp(scale*q_i.k_j)
 *            over the visible keys j.
 *   B, H, Hkv, N, d   sizes; d in {64, 128} for bf16, d == 128 for fp8.
 *                     Any N >= 1 (ragged tails are masked).
 *   causal   0 or non-zero (lower-triangular: key j <= query i).
 *   scale    multiplies Q K^T; any finite value (0 and negative included).
 *   dtype    fa_dtype_t.  FA_DTYPE_FP8_E4M3 here means all three descale
 *            factors are 1; use fa_fwd_fp8 to pass per-tensor descales.
 *   stream   hipStream_t or NULL.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int Hkv, int N, int d, int causal, float scale,
           int dtype, void* stream);

/*
 * fa_fwd_fp8 -- attention forward on per-tensor-scaled OCP e4m3 inputs, the
 * FP8 path of the FlashAttention-3 summary (GeekNews), sections «Principais
 * tecnologias do FlashAttention-3» and «Novos recursos de hardware da GPU
 * Hopper»: tensor X is represented by codes x8 and a descale factor
 * delta_X with X ~= decode(x8) * delta_X.
 *   q8, k8, v8   device e4m3 codes, layouts as above.
 *   o, lse       as for fa_fwd (o is bfloat16).  lse is formed from the
 *                unrounded fp32 weights, but the e4m3 matrix cores do not
 *                add their 64 products exactly in fp32 (a product is
 *                truncated to the alignment of the largest in its group of
 *                eight), so a score next to an outlier product is off by
 *                about 2^-14 of that product: |lse - exact| stays within
 *                5e-2 on inputs with 0.1% outliers x20 (about 1e-3
 *                without outliers).
 *   descale_qkv  device float[3] = {delta_Q, delta_K, delta_V}, read by the
 *                kernel (no host synchronisation), or NULL for {1, 1, 1}.
 *   d            must be 128.  Other arguments as for fa_fwd.
 * Computes O = softmax(scale * dQ * dK * Q8 K8^T) (dV * V8) with Q8/K8/V8 the
 * decoded codes; P is rounded to e4m3 before the P V product.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o,
               float* lse, int B, int H, int Hkv, int N, int d, int causal,
               float scale, const float* descale_qkv, void* stream);

/*
 * fa_fwd_fp8_exp2_fma -- fa_fwd_fp8 with part of the softmax's
 * exponentials computed on the FMA pipe instead of the exponential
 * instruction, the technique of the FlashAttention-4 article
 * («Оптимизируйте производительность с FlashAttention-4», paragraph 3).
 * The software 2^x (fa_exp2_fma below) is within 7.5e-5 relative of 2^x.
 *   fma_pairs  how many of the 16 pairs of weights each lane forms per
 *              64-key tile use it: 0 (same kernel as fa_fwd_fp8), 4, 8 or
 *              16; other values give FA_ERR_UNSUPPORTED (checked with d).
 *   Other arguments, results and accuracy as for fa_fwd_fp8.  On this chip
 *   the option is slower (eight vector instructions against one
 *   v_exp_f32, which shares their issue), so fa_fwd_fp8 does not use it.
 */
int fa_fwd_fp8_exp2_fma(const void* q8, const void* k8, const void* v8,
                        void* o, float* lse, int B, int H, int Hkv, int N,
                        int d, int causal, float scale,
                        const float* descale_qkv, int fma_pairs,
                        void* stream);

/*
 * fa_exp2_fma -- y[i] = 2^x[i] by the FMA-pipe exponential of
 * fa_fwd_fp8_exp2_fma (the same device function), for testing it.  Range
 * reduction x = n + f, n = rint(x), f in [-1/2, 1/2] (exact in base 2), a
 * degree-3 minimax polynomial for 2^f (Remez), 2^n added to the exponent.
 *   x, y     device float arrays of n elements, 4-byte aligned (x read
 *            only, y written; they may be the same array).
 *   n        >= 0 (0 enqueues nothing).
 *   Accuracy: for -125 <= x <= 127, |y / 2^x - 1| <= 7.5e-5; x < -125
 *   (-inf included) gives about 2.35e-38 (2^-125 times p(0)) instead of
 *   a smaller value; x > 127 or NaN is outside the contract.
 *   Errors: FA_ERR_INVALID_ARGUMENT (null pointer, n < 0),
 *   FA_ERR_MISALIGNED, FA_ERR_HIP.
 */
int fa_exp2_fma(const float* x, float* y, long long n, void* stream);

/*
 * fa_bwd -- gradients of the bf16 forward: dQ, dK, dV for a given dO.
 *   The pages name recomputation as the way FlashAttention avoids storing
 *   the attention matrix (FlashAttention-3 summary, GeekNews, section
 *   «Resumo do FlashAttention») and shared-memory traffic as the backward
 *   pass's bottleneck (FlashAttention-4 page, smntcn.com, paragraph 2); the
 *   formulas are the exact gradients of the forward's definition, with the
 *   softmax recomputed from the forward's LSE:
 *       P = exp(scale Q K^T - LSE), dV = P^T dO, dP = dO V^T,
 *       D_i = dO_i . O_i, dS = P * (dP - D), dQ = scale dS K,
 *       dK = scale dS^T Q; with GQA, dK and dV sum over each KV head's
 *       query heads.
 *   q, k, v, o, lse   the forward's inputs and outputs (read only): bf16
 *                     [B][H][N][d] / [B][Hkv][N][d], lse float [B][H][N].
 *   dout      device, bfloat16 [B][H][N][d] (read only): dL/dO.
 *   dq        device, bfloat16 [B][H][N][d] (written).
 *   dk, dv    device, bfloat16 [B][Hkv][N][d] (written).
 *   workspace device, float [B][H][N][2], caller-owned scratch (written):
 *             {LSE * log2(e), D} per query row.  Not an output.
 *   d         must be 128.  B, H, Hkv, N, causal, scale as for fa_fwd.
 *   stream    hipStream_t or NULL; three kernels are enqueued on it.
 *   Errors as for fa_fwd; a null dout, dq, dk, dv or workspace is
 *   FA_ERR_INVALID_ARGUMENT, a misaligned one FA_ERR_MISALIGNED.
 *   Deterministic: no atomics, the same inputs give the same bits.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           float* workspace, int B, int H, int Hkv, int N, int d, int causal,
           float scale, void* stream);

/*
 * fa_fwd_splitkv -- bf16 forward for Nq queries against Nk keys (decode and
 *   other short-query shapes), with the key range split across workgroups
 *   and the partial results merged by their log-sum-exp:
 *       LSE = ln sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s.
 *   The pages motivate it as long-context processing (FlashAttention-3
 *   summary, GeekNews, sections «Importância do Attention» and «Melhorias de
 *   desempenho do FlashAttention-3»).
 *   q         device, bfloat16 [B][H][Nq][d] (read only).
 *   k, v      device, bfloat16 [B][Hkv][Nk][d] (read only).
 *   o         device, bfloat16 [B][H][Nq][d] (written).
 *   lse       device, float [B][H][Nq] (written, natural log; -inf for a
 *             query that sees no key, whose o row is 0).
 *   causal    non-zero: bottom-right alignment, query i sees key j iff
 *             j <= i + Nk - Nq.
 *   num_splits  1 .. 256; fa_splitkv_num_splits() gives a good value.
 *   workspace device, float, num_splits * B * H * Nq * (d + 1) elements,
 *             caller-owned scratch (written): the splits' partial outputs
 *             and LSEs.  Not an output.
 *   d         must be 128.  Other arguments as for fa_fwd.
 *   Errors as for fa_fwd; num_splits out of range or a null workspace is
 *   FA_ERR_INVALID_ARGUMENT, a misaligned workspace FA_ERR_MISALIGNED.
 *   Two kernels are enqueued on `stream`.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int H, int Hkv, int Nq, int Nk, int d,
                   int causal, float scale, int num_splits, float* workspace,
                   void* stream);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate
 *   device memory (code under HIP graph capture, tight serving loops,
 *   harnesses that forbid hipMalloc): the same kernels and results, with
 *   the workspace replaced by a fixed scratch that the library holds on
 *   every GPU it runs on until the process ends (4194304 floats, 16 MiB).
 *   The call allocates nothing; its first call on a device looks up that
 *   device's scratch address (hipGetSymbolAddress, no allocation).
 *   Arguments as for fa_fwd_splitkv without workspace; the current device
 *   must be the stream's.  num_splits * B * H * Nq * (d + 1) must be at
 *   most 4194304, else FA_ERR_WORKSPACE (after the other checks, before
 *   anything is enqueued).  All calls on one GPU share its scratch: calls
 *   that overlap on one GPU (other streams, other threads) race; calls in
 *   order on one stream do not.  Nothing in the scratch needs clearing.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v,
                           void* o, float* lse, int B, int H, int Hkv, int Nq,
                           int Nk, int d, int causal, float scale,
                           int num_splits, void* stream);

/*
 * fa_splitkv_num_splits -- the split count fa_fwd_splitkv is tuned for on
 *   this GPU for the given sizes (about 1024 waves of work, one round at
 *   five waves per CU; at least 4 32-key tiles per split, at most 256).
 *   Returns 0 for invalid sizes.
 *   Host-only; enqueues nothing.
 */
int fa_splitkv_num_splits(int B, int H, int Hkv, int Nq, int Nk);

/*
 * fa_fwd_varlen -- bf16 forward over a packed batch of sequences of
 *   different lengths, with an optional sliding window (variable masking).
 *   The FlashAttention-3 summary (GeekNews), section «Comentários no Hacker
 *   News», asks about both (variable masking being slow, and sliding-window
 *   attention).  Sequences never see each other; within sequence b, with
 *   Nq_b, Nk_b its lengths and off = Nk_b - Nq_b (bottom-right alignment),
 *   query i sees key j iff (window_left < 0 or j >= i + off - window_left)
 *   and (window_right < 0 or j <= i + off + window_right); causal != 0 is
 *   window_right = 0.  Rows that see no key get o = 0 and lse = -inf.
 *   q, o      device, bfloat16 [H][total_q][d] (rows of all sequences
 *             packed per head; q read only, o written).
 *   k, v      device, bfloat16 [Hkv][total_k][d] (read only).
 *   lse       device, float [H][total_q] (written, natural log).
 *   cu_seqlens_q, cu_seqlens_k  device, int32 [B + 1]: sequence b owns rows
 *             [cu[b], cu[b+1]).  Read by the kernel: a sequence whose rows
 *             fall outside [0, total) is skipped and its outputs are left
 *             unwritten.
 *   max_seqlen_q  the longest query sequence (the grid is sized from it;
 *             the library cannot read cu_seqlens_q without a synchronisation).
 *             A smaller value computes each sequence's rows below it; rows
 *             at or past it rounded up to a multiple of 256 are not written.
 *   total_q, total_k  at most 2^29 (FA_ERR_INVALID_ARGUMENT above).
 *   window_left, window_right  >= -1 (-1 = unbounded); any width reaching
 *             past every sequence (window_left >= total_k, window_right >=
 *             total_q) is the unbounded window.
 *   d must be 128; H, Hkv, scale as for fa_fwd.  Errors as for fa_fwd;
 *   lse and the cu_seqlens arrays need 4-byte alignment.  One kernel is
 *   enqueued on `stream`.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                  float* lse, const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int B, int H, int Hkv, int total_q, int total_k,
                  int max_seqlen_q, int d, int causal, int window_left,
                  int window_right, float scale, void* stream);

/*
 * fa_fwd_masked -- bf16 forward under an arbitrary visibility mask.  The
 *   FlashAttention-3 summary (GeekNews), section «Comentários no Hacker
 *   News», reports FlashAttention being much slower with arbitrary masks.
 *   Query i of (batch b, query head h) sees key j iff bit j % 32 of word
 *   mask[b * mask_batch_stride + h * mask_head_stride + i * W + j / 32] is
 *   set, W = ceil(Nk / 32); the softmax runs over the visible keys only and
 *   a row that sees no key gets o = 0 and lse = -inf.  Work follows the
 *   mask: a 64-key tile is loaded and computed for a block of 128 query
 *   rows only if one of them sees one of its keys, and its mask words are
 *   only read if some row of the block does not see all of them.
 *   q, o      device, bfloat16 [B][H][Nq][d] (q read only, o written).
 *   k, v      device, bfloat16 [B][Hkv][Nk][d] (read only).
 *   lse       device, float [B][H][Nq] (written, natural log).
 *   mask      device, uint32 words, 4-byte aligned, read only; each
 *             (b, h) slice is Nq rows of W words.  Bits past Nk are ignored.
 *   mask_batch_stride, mask_head_stride  in words, >= 0; 0 shares one mask
 *             slice across batches or heads.
 *   Nk at most 262144 (FA_ERR_UNSUPPORTED above); d must be 128; H, Hkv,
 *   scale as for fa_fwd.  Errors as for fa_fwd; lse needs 4-byte alignment.
 *   One kernel is enqueued on `stream`.
 */
int fa_fwd_masked(const void* q, const void* k, const void* v, void* o,
                  float* lse, const unsigned int* mask,
                  long long mask_batch_stride, long long mask_head_stride,
                  int B, int H, int Hkv, int Nq, int Nk, int d, float scale,
                  void* stream);

/*
 * fa_fp8_quantize -- optional random-sign Hadamard rotation of each row, then
 * per-tensor OCP e4m3 quantisation ("incoherent processing" of the
 * FlashAttention-3 summary, section «Baixa precisão: redução do erro de
 * quantização com processamento incoerente»).
 *   x             device float [rows][d] (read only).
 *   x8            device uint8 [rows][d] (written): e4m3 codes of
 *                 x' * (448 / amax), rounded to nearest even in fp32 and
 *                 saturated to +-448, where x' = x diag(s) H_d / sqrt(d) if
 *                 signs are given (H_d the Sylvester Hadamard matrix) and
 *                 x' = x otherwise, and amax = max |x'| over the tensor.
 *   amax_descale  device float[2] (written): {amax, amax / 448}; amax = 0
 *                 gives a descale of 1.  Element 1 is the delta to pass to
 *                 fa_fwd_fp8.
 *   rows, d       rows >= 1, d == 128.
 *   signs_host    host array of d int8 values, each +1 or -1, or NULL for no
 *                 rotation.  Q and K must be rotated with the same signs (the
 *                 rotation is orthonormal, so Q K^T is unchanged); V is not
 *                 rotated.
 *   stream        hipStream_t or NULL.  Three kernels are enqueued in order:
 *                 clear amax, reduce amax, quantise.
 * Errors as listed above; signs other than +-1 give FA_ERR_INVALID_ARGUMENT.
 */
int fa_fp8_quantize(const float* x, void* x8, float* amax_descale,
                    long long rows, int d, const signed char* signs_host,
                    void* stream);

/* Static description of a status code; never NULL. */
const char* fa_status_string(int status);

/* hipError_t behind the most recent FA_ERR_HIP returned on this thread
 * (0 if none). */
int fa_last_hip_error(void);

/* Library ABI version (major * 100 + minor). */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
