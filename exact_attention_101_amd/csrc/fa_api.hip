// C ABI of libfa.so: argument validation, kernel selection and launch on the
// caller's stream.  Declarations and the contract live in include/fa.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_common.h"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace fa {
hipError_t launch_fwd_bf16(FwdArgs a, int d, bool causal, hipStream_t stream);
hipError_t launch_fwd_fp8(FwdArgs a, bool causal, int fma_pairs,
                          hipStream_t stream);
hipError_t launch_exp2_fma(const float* x, float* y, long long n,
                           hipStream_t stream);
hipError_t launch_bwd_bf16(BwdArgs a, bool causal, hipStream_t stream);
hipError_t launch_splitkv_bf16(SplitArgs a, bool causal, hipStream_t stream);
hipError_t splitkv_scratch(float** out);
int splitkv_auto_splits(int B, int H, int Hkv, int Nq, int Nk);
hipError_t launch_fwd_varlen_bf16(FwdArgs a, int max_q, hipStream_t stream);
hipError_t launch_varlen_bf16(VarlenArgs a, hipStream_t stream);
hipError_t launch_fwd_masked_bf16(FwdArgs a, hipStream_t stream);
hipError_t launch_fp8_quantize(const float* x, uint8_t* x8, float* amax_descale,
                               long long rows, uint64_t sign_lo,
                               uint64_t sign_hi, bool rotate,
                               hipStream_t stream);
}  // namespace fa

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  g_last_hip_error = static_cast<int>(e);
  return FA_ERR_HIP;
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// a * b * c > limit, for positive ints, without overflowing (the product of
// three ints can pass 2^63).
bool product_exceeds(int a, int b, int c, long long limit) {
  const long long ab = static_cast<long long>(a) * b;   // < 2^62
  return ab > limit / c;
}

// Checks shared by both forward entry points, in the documented order.
int check_fwd(const void* q, const void* k, const void* v, const void* o,
              const void* lse, int B, int H, int Hkv, int N, int d,
              int causal, float scale, int d_ok) {
  (void)causal;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0 || d <= 0)
    return FA_ERR_INVALID_ARGUMENT;
  if (H % Hkv != 0) return FA_ERR_INVALID_ARGUMENT;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARGUMENT;
  // Element counts must fit comfortably in 64 bits; B*H*N must fit in int
  // arithmetic on the device side (per-head offsets are 64-bit).
  if (product_exceeds(B, H, N, 1LL << 40)) return FA_ERR_INVALID_ARGUMENT;
  if (!d_ok) return FA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(lse))
    return FA_ERR_MISALIGNED;
  return FA_OK;
}

fa::FwdArgs make_args(const void* q, const void* k, const void* v, void* o,
                      float* lse, int B, int H, int Hkv, int N, float scale) {
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.descale = nullptr;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.group = H / Hkv;
  a.scale = scale;
  a.neg = scale < 0.f;
  // Scores enter exp2 as S * c, c = |scale| * log2(e).  c is floored at
  // 1e-30 so that a masked score (-inf) always gives p = 0; for |scale| that
  // small every visible score maps to exp2(~0) = 1 in fp32 either way.
  a.c = fmaxf(fabsf(scale) * 1.4426950408889634f, 1e-30f);
  return a;
}

}  // namespace

FA_EXPORT int fa_fwd(const void* q, const void* k, const void* v, void* o,
                     float* lse, int B, int H, int Hkv, int N, int d,
                     int causal, float scale, int dtype, void* stream) {
  if (dtype == FA_DTYPE_FP8_E4M3) {
    return fa_fwd_fp8(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale, nullptr,
                      stream);
  }
  const int st = check_fwd(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale,
                           dtype == FA_DTYPE_BF16 && (d == 64 || d == 128));
  if (st != FA_OK) return st;
  fa::FwdArgs a = make_args(q, k, v, o, lse, B, H, Hkv, N, scale);
  return hip_status(fa::launch_fwd_bf16(a, d, causal != 0,
                                        static_cast<hipStream_t>(stream)));
}

FA_EXPORT int fa_fwd_fp8(const void* q8, const void* k8, const void* v8,
                         void* o, float* lse, int B, int H, int Hkv, int N,
                         int d, int causal, float scale,
                         const float* descale_qkv, void* stream) {
  const int st = check_fwd(q8, k8, v8, o, lse, B, H, Hkv, N, d, causal, scale,
                           d == 128);
  if (st != FA_OK) return st;
  if (descale_qkv && (reinterpret_cast<uintptr_t>(descale_qkv) & 3u))
    return FA_ERR_MISALIGNED;
  fa::FwdArgs a = make_args(q8, k8, v8, o, lse, B, H, Hkv, N, scale);
  a.descale = descale_qkv;
  return hip_status(fa::launch_fwd_fp8(a, causal != 0, 0,
                                       static_cast<hipStream_t>(stream)));
}

FA_EXPORT int fa_fwd_fp8_exp2_fma(const void* q8, const void* k8,
                                  const void* v8, void* o, float* lse, int B,
                                  int H, int Hkv, int N, int d, int causal,
                                  float scale, const float* descale_qkv,
                                  int fma_pairs, void* stream) {
  const int st = check_fwd(q8, k8, v8, o, lse, B, H, Hkv, N, d, causal, scale,
                           d == 128 && (fma_pairs == 0 || fma_pairs == 4 ||
                                        fma_pairs == 8 || fma_pairs == 16));
  if (st != FA_OK) return st;
  if (descale_qkv && (reinterpret_cast<uintptr_t>(descale_qkv) & 3u))
    return FA_ERR_MISALIGNED;
  fa::FwdArgs a = make_args(q8, k8, v8, o, lse, B, H, Hkv, N, scale);
  a.descale = descale_qkv;
  return hip_status(fa::launch_fwd_fp8(a, causal != 0, fma_pairs,
                                       static_cast<hipStream_t>(stream)));
}

FA_EXPORT int fa_exp2_fma(const float* x, float* y, long long n,
                          void* stream) {
  if (!x || !y || n < 0) return FA_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(x) & 3u) ||
      (reinterpret_cast<uintptr_t>(y) & 3u))
    return FA_ERR_MISALIGNED;
  return hip_status(
      fa::launch_exp2_fma(x, y, n, static_cast<hipStream_t>(stream)));
}

FA_EXPORT int fa_bwd(const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, float* workspace, int B,
                     int H, int Hkv, int N, int d, int causal, float scale,
                     void* stream) {
  if (!o || !dout || !dq || !dk || !dv || !workspace)
    return FA_ERR_INVALID_ARGUMENT;
  const int st = check_fwd(q, k, v, o, lse, B, H, Hkv, N, d, causal, scale,
                           d == 128);
  if (st != FA_OK) return st;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || !aligned16(workspace))
    return FA_ERR_MISALIGNED;
  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws = workspace;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.N = N;
  a.group = H / Hkv;
  a.scale = scale;
  a.c = scale * 1.4426950408889634f;
  return hip_status(
      fa::launch_bwd_bf16(a, causal != 0, static_cast<hipStream_t>(stream)));
}

FA_EXPORT int fa_splitkv_num_splits(int B, int H, int Hkv, int Nq, int Nk) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || H % Hkv != 0)
    return 0;
  return fa::splitkv_auto_splits(B, H, Hkv, Nq, Nk);
}

namespace {

// Checks shared by the two split-KV entry points, in the documented order
// (the workspace pointer, when there is one, is checked by the caller).
int check_splitkv(const void* q, const void* k, const void* v, const void* o,
                  const void* lse, int B, int H, int Hkv, int Nq, int Nk,
                  int d, float scale, int num_splits) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0)
    return FA_ERR_INVALID_ARGUMENT;
  if (H % Hkv != 0 || !isfinite(scale)) return FA_ERR_INVALID_ARGUMENT;
  if (num_splits < 1 || num_splits > fa::SPLITKV_MAX_SPLITS)
    return FA_ERR_INVALID_ARGUMENT;
  if (product_exceeds(B, H, Nq, 1LL << 40) ||
      product_exceeds(B, Hkv, Nk, 1LL << 40))
    return FA_ERR_INVALID_ARGUMENT;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(lse))
    return FA_ERR_MISALIGNED;
  return FA_OK;
}

int run_splitkv(const void* q, const void* k, const void* v, void* o,
                float* lse, int B, int H, int Hkv, int Nq, int Nk, int causal,
                float scale, int num_splits, float* workspace, void* stream) {
  fa::SplitArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.splits = num_splits;
  a.c = scale * 1.4426950408889634f;
  const long long rows = static_cast<long long>(B) * H * Nq;
  a.ws_o = workspace;
  a.ws_lse = workspace + rows * num_splits * 128;
  return hip_status(fa::launch_splitkv_bf16(a, causal != 0,
                                            static_cast<hipStream_t>(stream)));
}

}  // namespace

FA_EXPORT int fa_fwd_splitkv(const void* q, const void* k, const void* v,
                             void* o, float* lse, int B, int H, int Hkv,
                             int Nq, int Nk, int d, int causal, float scale,
                             int num_splits, float* workspace, void* stream) {
  if (!workspace) return FA_ERR_INVALID_ARGUMENT;
  const int st = check_splitkv(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale,
                               num_splits);
  if (st != FA_OK) return st;
  if (!aligned16(workspace)) return FA_ERR_MISALIGNED;
  return run_splitkv(q, k, v, o, lse, B, H, Hkv, Nq, Nk, causal, scale,
                     num_splits, workspace, stream);
}

FA_EXPORT int fa_fwd_splitkv_noalloc(const void* q, const void* k,
                                     const void* v, void* o, float* lse,
                                     int B, int H, int Hkv, int Nq, int Nk,
                                     int d, int causal, float scale,
                                     int num_splits, void* stream) {
  const int st = check_splitkv(q, k, v, o, lse, B, H, Hkv, Nq, Nk, d, scale,
                               num_splits);
  if (st != FA_OK) return st;
  // rows <= 2^40 and num_splits <= 256 after the checks: no overflow.
  const long long rows = static_cast<long long>(B) * H * Nq;
  const long long need = rows * num_splits * (d + 1);
  if (need > fa::SPLITKV_SCRATCH_FLOATS) return FA_ERR_WORKSPACE;
  float* ws = nullptr;
  const hipError_t e = fa::splitkv_scratch(&ws);
  if (e != hipSuccess) return hip_status(e);
  return run_splitkv(q, k, v, o, lse, B, H, Hkv, Nq, Nk, causal, scale,
                     num_splits, ws, stream);
}

FA_EXPORT int fa_fwd_varlen(const void* q, const void* k, const void* v,
                            void* o, float* lse, const int* cu_seqlens_q,
                            const int* cu_seqlens_k, int B, int H, int Hkv,
                            int total_q, int total_k, int max_seqlen_q, int d,
                            int causal, int window_left, int window_right,
                            float scale, void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k)
    return FA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || Hkv <= 0 || total_q <= 0 || total_k <= 0 ||
      max_seqlen_q <= 0 || d <= 0)
    return FA_ERR_INVALID_ARGUMENT;
  if (H % Hkv != 0 || !isfinite(scale) || window_left < -1 ||
      window_right < -1)
    return FA_ERR_INVALID_ARGUMENT;
  if (static_cast<long long>(H) * total_q > (1LL << 40) ||
      total_q > fa::VARLEN_MAX_ROWS || total_k > fa::VARLEN_MAX_ROWS)
    return FA_ERR_INVALID_ARGUMENT;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return FA_ERR_MISALIGNED;
  // A window at least as wide as every sequence is the unbounded one: with
  // query i of a sequence of NQ queries and NK keys seeing key j iff
  // i + off - left <= j <= i + off + right (off = NK - NQ, 0 <= j < NK),
  // left >= NK - 1 or right >= NQ - 1 hides nothing, and NK <= total_k,
  // NQ <= total_q.  Clamping keeps the kernels' i + off +- window sums
  // within int range for any window the caller passes.
  if (window_left >= total_k) window_left = -1;
  int right = causal ? 0 : window_right;
  if (right >= total_q) right = -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // Windows bounded on both sides and narrower than VARLEN_NARROW keys go
  // to the 128-row kernel, whose waves skip the tiles outside their own
  // rows' windows; everything else to the pipelined forward kernel, whose
  // 256-row workgroups stream W + 256 keys for a window of W.
  if (window_left >= 0 && right >= 0 &&
      window_left + right < fa::VARLEN_NARROW) {
    fa::VarlenArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.B = B;
    a.H = H;
    a.Hkv = Hkv;
    a.group = H / Hkv;
    a.total_q = total_q;
    a.total_k = total_k;
    a.max_q = max_seqlen_q;
    a.left = window_left;
    a.right = right;
    a.c = scale * 1.4426950408889634f;
    return hip_status(fa::launch_varlen_bf16(a, st));
  }
  fa::FwdArgs a = make_args(q, k, v, o, lse, B, H, Hkv, 0, scale);
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  a.left = window_left;
  a.right = right;
  return hip_status(fa::launch_fwd_varlen_bf16(a, max_seqlen_q, st));
}

FA_EXPORT int fa_fwd_masked(const void* q, const void* k, const void* v,
                            void* o, float* lse, const unsigned int* mask,
                            long long mask_batch_stride,
                            long long mask_head_stride, int B, int H, int Hkv,
                            int Nq, int Nk, int d, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse || !mask) return FA_ERR_INVALID_ARGUMENT;
  if (B <= 0 || H <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0)
    return FA_ERR_INVALID_ARGUMENT;
  if (H % Hkv != 0 || !isfinite(scale) || mask_batch_stride < 0 ||
      mask_head_stride < 0)
    return FA_ERR_INVALID_ARGUMENT;
  if (product_exceeds(B, H, Nq, 1LL << 40) ||
      product_exceeds(B, Hkv, Nk, 1LL << 40))
    return FA_ERR_INVALID_ARGUMENT;
  if (d != 128 || Nk > fa::MASK_MAX_NK) return FA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) ||
      (reinterpret_cast<uintptr_t>(mask) & 3u))
    return FA_ERR_MISALIGNED;
  fa::FwdArgs a = make_args(q, k, v, o, lse, B, H, Hkv, Nq, scale);
  a.total_q = Nq;
  a.total_k = Nk;
  a.mask = mask;
  a.mask_bs = mask_batch_stride;
  a.mask_hs = mask_head_stride;
  return hip_status(
      fa::launch_fwd_masked_bf16(a, static_cast<hipStream_t>(stream)));
}

FA_EXPORT int fa_fp8_quantize(const float* x, void* x8, float* amax_descale,
                              long long rows, int d,
                              const signed char* signs_host, void* stream) {
  if (!x || !x8 || !amax_descale) return FA_ERR_INVALID_ARGUMENT;
  if (rows <= 0 || d <= 0 || rows > (1LL << 40)) return FA_ERR_INVALID_ARGUMENT;
  uint64_t lo = 0, hi = 0;
  if (signs_host) {
    for (int i = 0; i < d && i < 128; ++i) {
      const int s = signs_host[i];
      if (s != 1 && s != -1) return FA_ERR_INVALID_ARGUMENT;
    }
  }
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(x8) ||
      (reinterpret_cast<uintptr_t>(amax_descale) & 3u))
    return FA_ERR_MISALIGNED;
  if (signs_host) {
    for (int i = 0; i < 128; ++i) {
      if (signs_host[i] < 0) {
        if (i < 64) lo |= (1ULL << i);
        else hi |= (1ULL << (i - 64));
      }
    }
  }
  return hip_status(fa::launch_fp8_quantize(
      x, static_cast<uint8_t*>(x8), amax_descale, rows, lo, hi,
      signs_host != nullptr, static_cast<hipStream_t>(stream)));
}

FA_EXPORT const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARGUMENT:
      return "FA_ERR_INVALID_ARGUMENT: null pointer, non-positive size, H not "
             "a multiple of Hkv, non-finite scale or oversized tensor";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: head dimension or dtype not supported";
    case FA_ERR_MISALIGNED:
      return "FA_ERR_MISALIGNED: tensor pointer not 16-byte aligned";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP launch failed";
    case FA_ERR_WORKSPACE:
      return "FA_ERR_WORKSPACE: num_splits * B * H * Nq * (d + 1) floats do "
             "not fit in the library's fixed scratch (4194304 floats); pass "
             "a workspace to fa_fwd_splitkv or use fewer splits";
    default: return "unknown fa status";
  }
}

FA_EXPORT int fa_last_hip_error(void) { return g_last_hip_error; }

FA_EXPORT int fa_version(void) { return 100; }
