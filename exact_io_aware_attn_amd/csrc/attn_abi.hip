// attn_abi.hip -- the extern "C" boundary: argument validation, kernel
// selection by (dtype, D) and error reporting.  Host code only.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"
#include "attn_common.h"
#include "attn_launch.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int run_forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale, int dtype,
                const float* dq, const float* dk, const float* dv, attn_stream_t stream) {
  g_last_error[0] = '\0';
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-NULL device pointers");
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1)
    return fail(ATTN_ERR_INVALID_ARG, "sizes must be >= 1 (B=%lld Hq=%lld Hkv=%lld Nq=%lld Nkv=%lld D=%lld)",
                (long long)B, (long long)Hq, (long long)Hkv, (long long)Nq, (long long)Nkv, (long long)D);
  if (Hq % Hkv != 0)
    return fail(ATTN_ERR_INVALID_ARG, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3)
    return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if ((dq && (reinterpret_cast<uintptr_t>(dq) & 3u)) || (dk && (reinterpret_cast<uintptr_t>(dk) & 3u)) ||
      (dv && (reinterpret_cast<uintptr_t>(dv) & 3u)))
    return fail(ATTN_ERR_INVALID_ARG, "descale pointers must be 4-byte aligned");

  const int elt = dtype == ATTN_F32 ? attn::ELT_F32 : dtype == ATTN_BF16 ? attn::ELT_BF16 : attn::ELT_FP8;
  const int64_t in_bytes = dtype == ATTN_F32 ? 4 : dtype == ATTN_BF16 ? 2 : 1;
  const int64_t out_bytes = dtype == ATTN_F32 ? 4 : 2;
  const int64_t lim = (int64_t)1 << 31;
  if (D > 1024 || D % 32 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "D=%lld unsupported: D must be a multiple of 32 in [32, 1024]", (long long)D);
  if (Nq * D * in_bytes >= lim || Nkv * D * in_bytes >= lim || Nq * D * out_bytes >= lim)
    return fail(ATTN_ERR_UNSUPPORTED, "a (batch, head) slab of q, k, v or o reaches 2^31 bytes");
  if (B * Hq > (int64_t)INT32_MAX || Nq > INT32_MAX || Nkv > INT32_MAX)
    return fail(ATTN_ERR_UNSUPPORTED, "B*Hq and sequence lengths must fit in 31 bits");
  if (B * Hq * ((Nq + 31) / 32) >= lim)
    return fail(ATTN_ERR_UNSUPPORTED, "grid too large: B*Hq*ceil(Nq/32) must be < 2^31");

  // The wide-head kernel (bf16, D a multiple of 64 in [192, 512]) and the
  // direct-to-LDS kernel (bf16, D = 64 or 128; e4m3, D = 64, 128 or 256) fold
  // the scale into one FMA before exp2 and take row maxima of the unscaled
  // scores, which needs scale > 0.  Every other D <= 256 case runs on the
  // generic tiled kernel and every other D > 256 case on the split-D kernels;
  // both scale before masking.
  attn::LaunchFn fn = nullptr;
  if (scale > 0.0f) fn = attn::wide_launcher(elt, (int)D);
  if (!fn && scale > 0.0f) fn = attn::pipe_launcher(elt, (int)D);
  if (!fn) fn = D <= 256 ? attn::tiled_launcher(elt, (int)D) : attn::splitd_launcher(elt, (int)D);
  if (!fn)
    return fail(ATTN_ERR_UNSUPPORTED, "no kernel for dtype=%d D=%lld (fp32: D%%32==0, D<=128; fp8: D%%64==0, "
                "D<=256; bf16: D%%32==0, D<=256, or D%%64==0 in [320, 1024])", dtype, (long long)D);

  attn::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Nq = (int)Nq;
  p.Nkv = (int)Nkv;
  p.group = (int)(Hq / Hkv);
  p.causal = causal ? 1 : 0;
  p.kv_off = (int)(Nkv - Nq);
  p.scale = scale;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  hipError_t err = fn(p, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(ATTN_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
             int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale, int dtype,
             attn_stream_t stream) {
  return run_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype, nullptr, nullptr, nullptr,
                     stream);
}

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                 int64_t Hkv, int64_t Nq, int64_t Nkv, int64_t D, int causal, float scale,
                 const float* descale_q, const float* descale_k, const float* descale_v, attn_stream_t stream) {
  return run_forward(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, ATTN_FP8_E4M3, descale_q, descale_k,
                     descale_v, stream);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_UNKNOWN_STATUS";
  }
}

const char* attn_last_error(void) { return g_last_error; }

int attn_version(void) { return 100; }

}  // extern "C"
